// octo_attend_decode: single-query attention over the packed OCTOPUS cache.
//
// Split-K flash decoding (OCTOPUS paper, arXiv 2605.21226, Sec. 3.6 and the
// App. A summary of the fused decode kernel) with the two contractions on
// the matrix cores.  Each workgroup scans one token range ("split") of one
// (batch, KV head) plane for the G query heads sharing that KV head.  Keys
// are never reconstructed in memory: each wavefront unpacks a 32-token block
// straight into MFMA operand registers,
//   u^_j = rho^_ji n^_ji   (Eq. 13: n^ the decoded direction of the code
//                           pair, rho^ the C_rho centroid),
// and the score of Eq. 13, gamma_j (R q) . u^_j, is one MFMA product of the
// block's u^ with the rotated queries.  With QJL the estimator of Sec. 3.6,
// gamma_j sqrt(pi/(2d)) gamma_r,j (R' R q) . sigma_j, is a second product
// with sigma_j = +-1 as an exact fp16 operand.  Values stay in the rotated
// frame: O += P (gamma_v u^_v), and R_v^T is applied once per head when the
// splits are merged.
//
// Precision.  The operands are split as x = hi + lo with hi, lo in fp16
// (hi = x rounded toward zero, lo = the fp32 residual rounded toward zero) and
// every product is formed as hi*hi + hi*lo + lo*hi (the key side with
// pre-split tables also adds lo*lo) with fp32 accumulation, about 2^-20
// relative: single fp16 operands are not accurate enough for the
// peaked softmax that outlier channels produce.  u^ is scaled by 64 (exact)
// so that the residuals stay in the fp16 normal range.
//
// Tables in LDS, built per workgroup from the codebooks.  The pre-split
// table holds 64 rho^ n^ for every (norm index, code pair), already split
// into fp16 hi/lo halves, at index rho K^2 + code pair, which is the
// triplet's field of the index stream as it is stored: unpacking a triplet
// is one field extraction and one LDS read.  Up to 1024 entries (b_dir <= 4 with b_nrm <= 2, or the
// uniform (2,2), (3,3)) two workgroups share a CU, each with its K and V
// tables; the 4-bit splits (5,3) and (4,4) take 4096 or 8192 entries, one
// table for K and V when they share their codebooks, in one eight-wave
// workgroup per CU.  Otherwise the table holds 64 n^ per code pair in fp32
// and rho^ is applied and split on the fly.

// MFMA lane layout of v_mfma_f32_16x16x32_f16 (L = lane):
//   A[i][k]: i = L % 16, k-slot 8 (L / 16) + e;  B[k][j]: j = L % 16, same k
//   D[i][j]: i = 4 (L / 16) + r, j = L % 16.
// Scores are S^T = U Q^T (tokens as rows), so each lane ends up with 4 keys
// of one query head, which is the A-operand layout P needs in O = P V.
// Key-side coordinates: lane group g = L / 16 of token row t owns the 11
// consecutive triplets 11 g .. 11 g + 10 (10 for g = 3), so that it reads
// only the few record words that cover them.  With pre-split tables, call m
// (eleven calls, two products each) takes triplet 11 g + m: slots 0-3 are
// its hi components (x, y, z, 0), slots 4-7 its lo components, which is the
// table entry as it stands, against the query's components repeated, hi in
// one product and lo in the other.  With fp32 tables, call (gi, c) slot e is
// component c of triplet 8 gi + e.
// With QJL, call k, slot e = sign bit 32 g + 8 k + e, one word of the sign
// record.
// Value-side columns: tile (grp, c), column j = component c of triplet
// 16 grp + j; slot e of lane group g = token 16 (e / 4) + 4 g + e % 4 of the
// 32-token block, matching the score layout.
//
// A second launch merges the splits by their log-sum-exp in split order and
// applies R_v^T, so results do not depend on scheduling.  (Merging inside the
// first launch, by the last workgroup of each plane to count itself in an
// arrival counter, was slower on every workload: with device-scope fences,
// which write back and invalidate a whole L2, the 32k call took twice as
// long; with device-scope stores and loads of the partials instead, the
// chain of round trips it adds at the end of the launch -- the stores, the
// count, the loads -- still outlasted the second launch.)
#include <math.h>

#include <cstring>
#include <mutex>

#include "octo_internal.h"

namespace octo {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef __fp16 fp16x2 __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWavesSmall = 4;        // waves per workgroup with small tables
constexpr int kWavesBig = 8;          // ... with the big pre-split table (one per CU)
constexpr int kBlock = 32;            // tokens per wavefront iteration
constexpr int kMaxG = 16;             // query heads per KV head (MFMA columns)
constexpr float kUScale = 64.0f;      // exact scale of u^ in the operands
constexpr float kInvSqrtD = 0.08838834764831845f;
constexpr float kQjlC = 1.2533141373155003f;  // sqrt(pi / 2)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLazy = 8.0f;                 // slack of the lazy running maximum (log2 units)
constexpr float kNormByte = 66.0f;            // exponent byte of value norms below 128
constexpr int kMaxSmallPre = 1024;    // largest pre-split table beside a second
                                      // workgroup on the CU (entries)

// Table modes: PRE holds rho^ n^ for every (code pair, norm index), split
// into fp16 hi/lo; FP32 holds n^ per code pair and rho^ is applied on the fly.
enum TableMode { kPre = 0, kFp32 = 1 };

struct DecodeArgs {
  const void* q;
  int q_bf16;
  int B, Hq, Hkv, G;
  const int* seq_lens;
  int max_len;
  float scale;
  Codebook kcb, vcb;   // C_xi, C_rho of K and of V
  int shared_tables;   // K and V use the same codebook values
  int v_group;         // 0, or the group size of the group-wise value codec
  uint64_t kseed, vseed;
  const uint32_t *k_idx, *kqjl, *v_idx;   // index streams, K sign stream
  const float *kgamma, *vgamma;
  const uint16_t* kgamma_r;
  int capacity;
  int n_split, split_len;
  int n_part;          // partials per (batch, query head): n_split
  float2* ws_ml;       // [B][Hq][n_part] (running max, normalizer)
  float* ws_acc;       // [B][Hq][n_part][128] rotated-frame value sums (x64)
  // octo_decode_step only (step = 1): (P_b, n_b) as the scan read them
  int step, window;
  const int* win_lens;                 // n_b, tokens in the ring before the step
  int2* snap;                          // [B] in the workspace
};

__device__ inline void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ inline uint32_t pk(fp16x2 h) { return __builtin_bit_cast(uint32_t, h); }

// (x & m) | c in one instruction, m and c held in vector registers (the
// compiler splits the expression when its constants need literal operands).
__device__ inline uint32_t and_or(uint32_t x, uint32_t m, uint32_t c) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "v"(m), "v"(c));
  return r;
}
// A constant materialized in a vector register.
__device__ inline uint32_t vreg(uint32_t c) {
  uint32_t r;
  asm volatile("v_mov_b32 %0, %1" : "=v"(r) : "i"(c));
  return r;
}

// x = hi + lo for 8 slots: hi rounded toward zero to fp16, lo the residual.
__device__ inline void split8(const float* x, half8& hi, half8& lo) {
  u32x4 h, l;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const fp16x2 a = __builtin_amdgcn_cvt_pkrtz(x[2 * k], x[2 * k + 1]);
    h[k] = pk(a);
    l[k] = pk(__builtin_amdgcn_cvt_pkrtz(x[2 * k] - (float)a.x, x[2 * k + 1] - (float)a.y));
  }
  hi = __builtin_bit_cast(half8, h);
  lo = __builtin_bit_cast(half8, l);
}

__device__ inline floatx4 mfma(const half8& a, const half8& b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// hi*hi + hi*lo + lo*hi
__device__ inline floatx4 mfma3(const half8& ah, const half8& al, const half8& bh,
                                const half8& bl, floatx4 c) {
  c = mfma(al, bh, c);
  c = mfma(ah, bl, c);
  return mfma(ah, bh, c);
}

__device__ inline float4 decode_dir(float xi, float eta) {
  // Eq. 6 / App. C.7: unfold, normalize onto S^2; scaled by 64.
  const float z = 1.0f - fabsf(xi) - fabsf(eta);
  float x = xi, y = eta;
  if (z < 0.0f) {
    x = (xi >= 0.0f ? 1.0f : -1.0f) * (1.0f - fabsf(eta));
    y = (eta >= 0.0f ? 1.0f : -1.0f) * (1.0f - fabsf(xi));
  }
  // |x| + |y| + |z| = 1 here, so the squared norm is at least 1/3
  const float n = kUScale * __builtin_amdgcn_rsqf(x * x + y * y + z * z);
  return make_float4(x * n, y * n, z * n, 0.0f);
}

// Pre-split entry of 64 rho^ n^: {hx|hy, hz|0, lx|ly, lz|0} as fp16 pairs.
__device__ inline uint4 presplit_entry(float4 n, float rho) {
  const float x = rho * n.x, y = rho * n.y, z = rho * n.z;
  const fp16x2 hxy = __builtin_amdgcn_cvt_pkrtz(x, y);
  const fp16x2 hz = __builtin_amdgcn_cvt_pkrtz(z, 0.0f);
  const fp16x2 lxy = __builtin_amdgcn_cvt_pkrtz(x - (float)hxy.x, y - (float)hxy.y);
  const fp16x2 lz = __builtin_amdgcn_cvt_pkrtz(z - (float)hz.x, 0.0f);
  return make_uint4(pk(hxy), pk(hz), pk(lxy), pk(lz));
}

// Operand pair of slots (e, e+1) for one component from two pre-split
// entries: low or high fp16 half of the same word of each.
__device__ inline uint32_t pair_lo(uint32_t e0, uint32_t e1) {
  return __builtin_amdgcn_perm(e1, e0, 0x05040100u);
}
__device__ inline uint32_t pair_hi(uint32_t e0, uint32_t e1) {
  return __builtin_amdgcn_perm(e1, e0, 0x07060302u);
}

// Operands of 8 slots from pre-split entries: component c hi / lo.
__device__ inline void operands_pre(const uint4* E, half8 (&hi)[3], half8 (&lo)[3]) {
  u32x4 hx, hy, hz, lx, ly, lz;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const uint4 a = E[2 * m], b = E[2 * m + 1];
    hx[m] = pair_lo(a.x, b.x);
    hy[m] = pair_hi(a.x, b.x);
    hz[m] = pair_lo(a.y, b.y);
    lx[m] = pair_lo(a.z, b.z);
    ly[m] = pair_hi(a.z, b.z);
    lz[m] = pair_lo(a.w, b.w);
  }
  hi[0] = __builtin_bit_cast(half8, hx);
  hi[1] = __builtin_bit_cast(half8, hy);
  hi[2] = __builtin_bit_cast(half8, hz);
  lo[0] = __builtin_bit_cast(half8, lx);
  lo[1] = __builtin_bit_cast(half8, ly);
  lo[2] = __builtin_bit_cast(half8, lz);
}

constexpr int kTriPerGroup = 11;      // triplets of one key-side lane group

// Record words that cover the bits of 11 triplets of FW bits from any shift.
constexpr int group_words(int FW) { return (31 + kTriPerGroup * FW + 31) / 32; }

// Value side: lane L (token L % 32, half L / 32) extracts the table indices of
// triplets 22 h .. 22 h + 21 of its token (the last one of half 1 is past the
// 43 and lands in a spare row).
constexpr int kValTri = 22;
constexpr int value_words(int FW) { return (31 + kValTri * FW + 31) / 32; }
constexpr int kIdxRow = 36;           // u16 per index row: 32 tokens + pad (bank spread)
constexpr int kIdxRows = 44;          // 43 triplets + the spare

// The global words of one 32-token block of a wavefront.  Key side: lane
// (col, grp4) holds, for tile kt, the record words of token 16 kt + col that
// cover the triplets of lane group grp4 (and word grp4 of its sign record);
// value side: lane L holds the record words of token L % 32 that cover
// triplets 22 (L / 32) .. + 21.
// With the group-wise value codec (VG = its group size) lane L instead holds
// words 2 k + L / 32 of token L % 32's value record (VW words).
template <int VB, int VG>
struct GroupRecord {
  static constexpr int G = kHeadDim / VG;             // groups per token
  static constexpr int WC = VB * kHeadDim / 32;       // code words
  static constexpr int W = group_record_words(VB, VG);
  static constexpr int kRows = WC + G;                // LDS rows: codes, fp16 scales, zeros
};

template <int BD, int BN, bool QJL, int VG = 0>
struct BlockWords {
  static constexpr int BT = 2 * BD + BN;            // bits of one triplet field
  static constexpr int WI = (kNTri * BT + 31) / 32;
  static constexpr int VW = VG ? group_record_words(BD - 1, VG) : 0;
  static constexpr int KWI = group_words(BT), KVI = VG ? (VW + 1) / 2 : value_words(BT);
  uint32_t iw[2][KWI], sw[2];
  uint32_t vi[KVI];
  float4 gk[2], gv[2];
  uint2 gr[2];
};

// Issues every load of the block at t0 (a multiple of 32, below the
// capacity, which is a multiple of 64, so that the 32 tokens share one
// 64-token tile) but the value norms.  Words of one token are 256 bytes
// apart: one base address per stream and immediate offsets; a group's window
// is clamped to the record (the words past its end only ever feed bits above
// the last field).
template <int BD, int BN, bool QJL, int VG>
__device__ inline void load_block(BlockWords<BD, BN, QJL, VG>& r, const DecodeArgs& a, size_t plane,
                                  int t0, int L) {
  using BW = BlockWords<BD, BN, QJL, VG>;
  constexpr int BT = BW::BT, WI = BW::WI;
  const int col = L & 15, grp4 = L >> 4, w0 = L >> 5, tk = L & 31;
  const int iwo = (kTriPerGroup * BT * grp4) >> 5;
  const size_t tile = plane * (size_t)(a.capacity >> 6) + (size_t)(t0 >> 6);
  const int tin = t0 & 63;
  const size_t gbase = plane * (size_t)a.capacity + (size_t)t0 + 4 * grp4;
#pragma unroll
  for (int kt = 0; kt < 2; ++kt) {
    const uint32_t* pi = a.k_idx + tile * (WI * 64) + tin + 16 * kt + col;
#pragma unroll
    for (int w = 0; w < BW::KWI; ++w) r.iw[kt][w] = pi[64 * min(iwo + w, WI - 1)];
    if (QJL) r.sw[kt] = a.kqjl[tile * (4 * 64) + tin + 16 * kt + col + 64 * grp4];
    r.gk[kt] = *reinterpret_cast<const float4*>(a.kgamma + gbase + 16 * kt);
    if (QJL) r.gr[kt] = *reinterpret_cast<const uint2*>(a.kgamma_r + gbase + 16 * kt);
  }
  if constexpr (VG != 0) {
    // value records: word 2 k + w0 of token tk (the spare slot of an odd
    // record re-reads its last word)
    const uint32_t* pvi = a.v_idx + tile * (BW::VW * 64) + tin + tk;
#pragma unroll
    for (int k = 0; k < BW::KVI; ++k) r.vi[k] = pvi[64 * min(2 * k + w0, BW::VW - 1)];
  } else {
    const int vwo = (kValTri * BT * w0) >> 5;
    const uint32_t* pvi = a.v_idx + tile * (WI * 64) + tin + tk;
#pragma unroll
    for (int w = 0; w < BW::KVI; ++w) r.vi[w] = pvi[64 * min(vwo + w, WI - 1)];
  }
}

// The value norms of the block at t0, loaded apart from the rest: the
// softmax still reads the current block's norms when the next block's
// words are requested, and a separate load keeps the two sets from being
// live at once (which costs register copies at the end of every iteration).
template <int BD, int BN, bool QJL, int VG>
__device__ inline void load_gv(BlockWords<BD, BN, QJL, VG>& r, const DecodeArgs& a, size_t plane,
                               int t0, int L) {
  if constexpr (VG != 0) return;           // the group codec has no value norms
  const size_t gbase = plane * (size_t)a.capacity + (size_t)t0 + 4 * (L >> 4);
#pragma unroll
  for (int kt = 0; kt < 2; ++kt)
    r.gv[kt] = *reinterpret_cast<const float4*>(a.vgamma + gbase + 16 * kt);
}

// ---------------------------------------------------------------- decode step
// The residual window of a decode step (octo_decode_step; the paper keeps the
// most recent tokens at native precision, OCTOPUS Sec. 4).  The scan is the
// one of octo_attend_decode over the packed prefix, and it copies each
// sequence's (P, n) to the workspace.  The merge launch then folds the
// window's native rows into each head's merge, and one more workgroup per
// sequence writes the new token to the ring, encodes the token leaving a
// full ring into its packed slot and updates the lengths (which nothing else
// in that launch reads: the other workgroups use the copy).
constexpr int kMaxWindow = 256;

// The encoder's tables for one codebook, in LDS: the decoded unit direction
// of every code pair with the pair's code (Eq. 6, App. C.7, normalized),
// padded by one clamped cell per side, so that the 3x3 neighbourhood of seed
// (sx, sy) is lut[(sx + dx) + KP (sy + dy)], dx, dy in 0..2; the C_xi cell
// boundaries padded with -inf and +inf; the C_rho boundaries.  The same
// arithmetic as encode_kernel's tables.  All threads of the workgroup build.
template <int BD, int BN>
__device__ void encoder_tables(const float* cx, const float* cr, floatx4* lut, float* midp,
                               float* mid_rho, int tid, int nthreads) {
  constexpr int K = 1 << BD, R = 1 << BN, KP = K + 2;
  for (int e = tid; e < KP * KP; e += nthreads) {
    const int ci = min(max(e % KP - 1, 0), K - 1), cj = min(max(e / KP - 1, 0), K - 1);
    const float xi = cx[ci], eta = cx[cj];
    const float z = 1.0f - fabsf(xi) - fabsf(eta);
    float x = xi, y = eta;
    if (z < 0.0f) {
      x = (xi >= 0.0f ? 1.0f : -1.0f) * (1.0f - fabsf(eta));
      y = (eta >= 0.0f ? 1.0f : -1.0f) * (1.0f - fabsf(xi));
    }
    const float n = fmaxf(sqrtf(x * x + y * y + z * z), 1e-20f);
    lut[e] = floatx4{x / n, y / n, z / n, __uint_as_float((uint32_t)(ci | (cj << BD)))};
  }
  if (tid <= K) midp[tid] = tid == 0 ? -INFINITY : tid == K ? INFINITY : 0.5f * (cx[tid - 1] + cx[tid]);
  if (tid < R - 1) mid_rho[tid] = 0.5f * (cr[tid] + cr[tid + 1]);
}

// One wavefront encodes one bf16 vector x[128] into slot t of a plane: the
// encoder of encode_kernel with the same decisions in the same arithmetic
// (Sec. 3.1-3.6), the 43 triplets spread over lanes 0..42 instead of one lane
// per vector, with the tables of encoder_tables.  u and fld are this
// wavefront's LDS scratch (129 floats, 43 words).
template <int BD, int BN>
__device__ void encode_one(const uint16_t* x, const floatx4* lut, const float* midp,
                           const float* mid_rho, const float* cr, uint64_t seed, int rounding,
                           bool qjl, uint32_t* idx, float* gamma, uint32_t* qjl_bits,
                           uint16_t* gamma_r, size_t plane, int cap, int t, float* u,
                           uint32_t* fld) {
  constexpr int K = 1 << BD, R = 1 << BN, FWD = 2 * BD, BT = FWD + BN, KP = K + 2;
  constexpr int WI = (kNTri * BT + 31) / 32;
  const int L = threadIdx.x & 63;
  // gamma, sign flip, rotation (Sec. 3.1)
  float a0 = bf16_to_f32(x[L]), a1 = bf16_to_f32(x[L + 64]);
  const float gam = sqrtf(wave_sum(fmaf(a0, a0, a1 * a1)));
  a0 *= splitmix_sign(seed, L);
  a1 *= splitmix_sign(seed, L + 64);
  wht128(a0, a1);
  const float scale = kInvSqrtD / fmaxf(gam, 1e-20f);
  u[L] = a0 * scale;
  u[L + 64] = a1 * scale;
  if (L == 0) u[128] = 0.0f;                          // the zero pad (Sec. 3.2)
  wave_sync();
  if (L < kNTri) {
    const float tx = u[3 * L], ty = u[3 * L + 1], tz = u[3 * L + 2];
    // Eq. 5 on the L1-normalized direction, sign(0) = +1
    const float inv_l1 = __builtin_amdgcn_rcpf(fmaxf(fabsf(tx) + fabsf(ty) + fabsf(tz), 1e-20f));
    const float px = tx * inv_l1, py = ty * inv_l1, pz = tz * inv_l1;
    float xi = px, eta = py;
    if (pz < 0.0f) {
      xi = (px >= 0.0f ? 1.0f : -1.0f) * (1.0f - fabsf(py));
      eta = (py >= 0.0f ? 1.0f : -1.0f) * (1.0f - fabsf(px));
    }
    // Lloyd seeds: the number of C_xi cell boundaries below (binary search)
    int sx = 0, sy = 0;
#pragma unroll
    for (int step = K >> 1; step > 0; step >>= 1) {
      if (xi > midp[sx + step]) sx += step;
      if (eta > midp[sy + step]) sy += step;
    }
    const floatx4* nbh = lut + sx + KP * sy;
    floatx4 nb = nbh[1 + KP];                          // the seed
    float sel;
    if (rounding == OCTO_ROUND_SCALAR) {
      sel = sqrtf(tx * tx + ty * ty + tz * tz);
    } else {
      // seed first, then the other eight neighbours row-major (dx outer);
      // only a strictly larger s replaces the incumbent (Sec. 3.5)
      float best = tx * nb.x + ty * nb.y + tz * nb.z;
#pragma unroll
      for (int dx = 0; dx < 3; ++dx)
#pragma unroll
        for (int dy = 0; dy < 3; ++dy) {
          if (dx == 1 && dy == 1) continue;
          const floatx4 n = nbh[dx + KP * dy];
          const float sv = tx * n.x + ty * n.y + tz * n.z;
          if (sv > best) {
            best = sv;
            nb = n;
          }
        }
      sel = best;
    }
    int ir = 0;
#pragma unroll
    for (int k = 0; k < R - 1; ++k) ir += sel > mid_rho[k] ? 1 : 0;
    fld[L] = __float_as_uint(nb.w) | ((uint32_t)ir << FWD);
    if (qjl) {
      // rotated-frame residual r = u - u^ over the real coordinates (Sec. 3.6)
      const float rho = cr[ir];
      u[3 * L] = tx - rho * nb.x;
      u[3 * L + 1] = ty - rho * nb.y;
      if (3 * L + 2 < kHeadDim) u[3 * L + 2] = tz - rho * nb.z;
    }
  }
  wave_sync();
  // pack: word w gathers the fields that overlap its 32 bits
  if (L < WI) {
    uint32_t word = 0u;
    const int i0 = 32 * L / BT, i1 = min(kNTri - 1, (32 * L + 31) / BT);
    for (int i = i0; i <= i1; ++i) {
      const int pos = i * BT - 32 * L;
      word |= pos >= 0 ? fld[i] << pos : fld[i] >> -pos;
    }
    idx[tile_word(plane, cap, t, L, WI)] = word;
  }
  if (L == 0) gamma[plane * cap + t] = gam;
  if (qjl) {
    // sigma = sign(H diag(s') r), gamma_r = fp16(||r||)
    float r0 = u[L], r1 = u[L + 64];
    const float rn = sqrtf(wave_sum(fmaf(r0, r0, r1 * r1)));
    r0 *= splitmix_sign(seed, kHeadDim + L);
    r1 *= splitmix_sign(seed, kHeadDim + L + 64);
    wht128(r0, r1);
    const uint64_t b0 = __ballot(r0 < 0.0f), b1 = __ballot(r1 < 0.0f);
    if (L < 4) {
      const uint64_t bb = L < 2 ? b0 : b1;
      qjl_bits[tile_word(plane, cap, t, L, 4)] = (uint32_t)(bb >> (32 * (L & 1)));
    }
    if (L == 0) gamma_r[plane * cap + t] = __builtin_bit_cast(uint16_t, (_Float16)rn);
  }
}

// A zero block standing in for the first block's speculative loads when the
// cache holds no tokens: 64 tokens of the widest record (words past the
// record's end are clamped to its last word).
constexpr int kZeroBlockWords = 64 * 40;
__device__ uint32_t g_zero_block[kZeroBlockWords];

template <int BD, int BN, bool QJL, int MODE, int NW, int VG = 0>
__global__ __launch_bounds__(64 * NW, 8 / NW) void decode_kernel(DecodeArgs a) {
  constexpr int kThreads = 64 * NW, kWaves = NW;
  constexpr int K = 1 << BD, R = 1 << BN, FWD = 2 * BD, BT = FWD + BN;
  constexpr bool PRE = MODE == kPre;                // pre-split (code, rho) table
  constexpr bool BIG = K * K * R > kMaxSmallPre;    // one shared table, one WG per CU
  constexpr int kTab = PRE ? K * K * R : K * K;     // entries per table (16 B each)
  // Small pre-split tables are stored in kCopies interleaved copies (entry
  // e of copy c at kCopies e + c; lane L reads copy L mod kCopies), at most
  // 32 KB a table: the 16 lanes that one LDS pass of a 16-byte gather serves
  // then read 16 different bank quads whatever their entries.
  constexpr int kCopies = !PRE || BIG ? 1 : (kTab * 16 * 16 <= 32768 ? 16 : 32768 / (kTab * 16));
  constexpr int kTabBytes = (VG || (PRE && BIG) ? 1 : 2) * kTab * 16 * kCopies;   // VG: the K table alone
  using GR = GroupRecord<(VG ? BD - 1 : 2), (VG ? VG : 32)>;            // the value record (VG)
  static_assert(BlockWords<BD, BN, QJL, VG>::WI <= kZeroBlockWords / 64 &&
                    BlockWords<BD, BN, QJL, VG>::VW <= kZeroBlockWords / 64,
                "the zero block covers a 64-token tile of every stream");
  static_assert(GR::kRows * 32 * 4 <= kIdxRows * kIdxRow * 2, "value records fit a wave's rows");
  constexpr int kRedBytes = kWaves * kMaxG * kHeadDim * 4;
  constexpr int kUnion = kTabBytes > kRedBytes ? kTabBytes : kRedBytes;

  // tables during the scan, the per-wave partial sums afterwards
  __shared__ __attribute__((aligned(16))) char smem[kUnion];
  __shared__ float crk[R], crv[R], cxk[K], cxv[K];
  // R q (then R' R q with QJL) during the set-up; the value-side table
  // indices of each wavefront's block in the scan
  constexpr int kQsBytes = kMaxG * 132 * 4, kIdxBytes = kWaves * kIdxRows * kIdxRow * 2;
  __shared__ __attribute__((aligned(16))) char qbuf[kQsBytes > kIdxBytes ? kQsBytes : kIdxBytes];
  float* qs = reinterpret_cast<float*>(qbuf);
  __shared__ float red_ml[kWaves * kMaxG * 2];
  // group codec: per-wave zero-point sums of each (head, group)
  __shared__ float red_z[VG ? kWaves * kMaxG * GR::G : 1];

  const int tid = threadIdx.x, L = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = L & 15, grp4 = L >> 4;
  const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int G = a.G;
  const size_t plane = (size_t)b * a.Hkv + g;
  // The big pre-split table serves K and V; small pre-split tables are
  // built twice (V's own copy even when the codebooks agree), so that the V
  // table sits at a constant offset that the LDS reads take as an
  // immediate.  fp32 tables are shared when the codebooks agree.
  uint4* tabk = reinterpret_cast<uint4*>(smem);
  uint4* tabv = PRE ? (BIG ? tabk : tabk + kTab * kCopies) : (a.shared_tables ? tabk : tabk + kTab);
  float* red_o = reinterpret_cast<float*>(smem);          // [wave][head][128]
  // this lane's copy of each table
  const uint4* tabk_l = tabk + (L & (kCopies - 1));
  const uint4* tabv_l = tabv + (L & (kCopies - 1));

  // ---- every global load of the prologue goes out first, none waiting for
  // another: codebooks, q, the first block and seq_lens.  The kernel
  // arguments their addresses need come in one batch of scalar loads (a
  // first use further down would wait for its own round trip).  The
  // codebooks are vector loads of the argument block, one value per lane;
  // the first block is loaded unconditionally (a block of the plane below
  // min(max_len, capacity), or a zero block when that is empty), so that the
  // compiler's counts of outstanding loads are exact and the table build
  // waits for the codebooks alone.
  const int cbl = min(L, kMaxXi + kMaxRho - 1);
  const float cb_k = reinterpret_cast<const float*>(&a.kcb)[cbl];
  const float cb_v = reinterpret_cast<const float*>(&a.vcb)[cbl];
  asm volatile("" ::"s"(a.q), "s"(a.k_idx), "s"(a.v_idx), "s"(a.kgamma), "s"(a.vgamma),
               "s"(a.seq_lens), "s"(a.max_len), "s"(a.capacity), "s"(a.split_len), "s"(a.Hq),
               "s"(a.G), "s"(a.Hkv), "s"(a.q_bf16));
  constexpr int kHeadsPerWave = kMaxG / kWaves;
  uint32_t qraw[kHeadsPerWave][2];                 // bf16 or fp32 bits
#pragma unroll
  for (int k = 0; k < kHeadsPerWave; ++k) {
    // heads past G read head G - 1 (unused): unconditional loads
    const int hh = min(wave + kWaves * k, G - 1);
    const size_t qo = ((size_t)b * a.Hq + (size_t)g * G + hh) * kHeadDim;
    const uint32_t* q32 = static_cast<const uint32_t*>(a.q);
    const uint16_t* q16 = static_cast<const uint16_t*>(a.q);
    qraw[k][0] = a.q_bf16 ? (uint32_t)q16[qo + L] : q32[qo + L];
    qraw[k][1] = a.q_bf16 ? (uint32_t)q16[qo + L + 64] : q32[qo + L + 64];
  }
  const int t_begin = split * a.split_len;
  int t0 = t_begin + wave * kBlock;
  BlockWords<BD, BN, QJL, VG> blk;
  if (!QJL) {
    const int lim = min(a.max_len, a.capacity);
    DecodeArgs f = a;
    size_t fplane = plane;
    int ft0 = min(t0, (lim - 1) & ~(kBlock - 1));
    if (lim <= 0) {                       // uniform: scalar selects, no branch
      f.k_idx = f.v_idx = g_zero_block;
      f.kgamma = f.vgamma = reinterpret_cast<const float*>(g_zero_block);
      f.capacity = 64;
      fplane = 0;
      ft0 = 0;
    }
    load_block(blk, f, fplane, ft0, L);
    load_gv(blk, f, fplane, ft0, L);
  }
  const int len_raw = __hip_atomic_load(a.seq_lens + b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const int win_raw = a.step ? __hip_atomic_load(a.win_lens + b, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT) : 0;

  // ---- tables: codebooks to LDS first, then the table entries
  if (tid < K) {
    cxk[tid] = cb_k;
    cxv[tid] = cb_v;
  }
  if (tid >= kMaxXi && tid < kMaxXi + R) {
    crk[tid - kMaxXi] = cb_k;
    crv[tid - kMaxXi] = cb_v;
  }
  lds_barrier();
  const int n_tables = VG ? 1 : (PRE || !a.shared_tables ? 2 : 1);
  // pre-split tables are rho-major, entry rho_index K^2 + code pair, so that
  // consecutive lanes write consecutive entries
  constexpr int KK = K * K;
  if (PRE && BIG) {
    // the (shared) table: each lane decodes the direction of its code pairs
    // once, in registers, and writes the entries of every norm index
    if constexpr (KK >= kThreads) {
      for (int c = tid; c < KK; c += kThreads) {
        const float4 n = decode_dir(cxk[c % K], cxk[c / K]);
#pragma unroll
        for (int r = 0; r < R; ++r) tabk[r * KK + c] = presplit_entry(n, crk[r]);
      }
    } else {
      constexpr int kSlices = kThreads / KK;        // lanes per code pair
      const int c = tid % KK;
      const float4 n = decode_dir(cxk[c % K], cxk[c / K]);
#pragma unroll
      for (int r = tid / KK; r < R; r += kSlices) tabk[r * KK + c] = presplit_entry(n, crk[r]);
    }
  } else if (PRE) {
    // small pre-split tables: one direction per (table, code pair), written
    // for every norm index
    for (int e = tid; e < n_tables * KK; e += kThreads) {
      const bool v = e >= KK;
      const int code = v ? e - KK : e;
      const float* cx = v ? cxv : cxk;
      const float* cr = v ? crv : crk;
      const float4 n = decode_dir(cx[code % K], cx[code / K]);
      uint4* t = tabk + (v ? kTab * kCopies : 0);
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const uint4 en = presplit_entry(n, cr[r]);
#pragma unroll
        for (int c = 0; c < kCopies; ++c) t[(r * KK + code) * kCopies + c] = en;
      }
    }
  } else {
    for (int e = tid; e < n_tables * kTab; e += kThreads) {
      const bool v = e >= kTab;
      const int i = v ? e - kTab : e;
      const float* cx = v ? cxv : cxk;
      const float4 n = decode_dir(cx[i % K], cx[i / K]);
      tabk[e] = make_uint4(__float_as_uint(n.x), __float_as_uint(n.y), __float_as_uint(n.z), 0u);
    }
  }
  // ---- q_rot = H diag(s) q / sqrt(d) for the G heads (rows >= G are zero),
  // times the softmax scale and log2(e): scores leave the MFMA in log2 units
  const float qscale = kInvSqrtD * a.scale * kLog2e;
  const float s_lo = splitmix_sign(a.kseed, L), s_hi = splitmix_sign(a.kseed, L + 64);
#pragma unroll
  for (int k = 0; k < kHeadsPerWave; ++k) {
    const int hh = wave + kWaves * k;
    const int qsh = a.q_bf16 ? 16 : 0;
    float q0 = __uint_as_float(qraw[k][0] << qsh) * s_lo;
    float q1 = __uint_as_float(qraw[k][1] << qsh) * s_hi;
    if (wave + kWaves * k < G)
      wht128(q0, q1);
    else
      q0 = q1 = 0.0f;                   // rows past G are zero
    qs[hh * 132 + L] = q0 * qscale;
    qs[hh * 132 + L + 64] = q1 * qscale;
  }
  lds_barrier();

  // Q^T operands (B), column col = head.  Pre-split tables: eleven calls m,
  // one per triplet 11 grp4 + m of the lane group; slot e = component e % 4
  // of that triplet (component 3 a zero pad), the same four values twice, so
  // that against the table entry {hi | lo} as it stands one call with the hi
  // operand and one with the lo operand give (hi + lo)(qh + ql).  fp32
  // tables: six calls m = (gi, c) = (m / 3, m % 3), slot e = component c of
  // triplet 8 gi + e.  Zero outside the group's triplets and the 128
  // coordinates.
  half8 qh[PRE ? kTriPerGroup : 6], ql[PRE ? kTriPerGroup : 6];
  if constexpr (PRE) {
#pragma unroll
    for (int m = 0; m < kTriPerGroup; ++m) {
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int c = e & 3;
        const int coord = 3 * (kTriPerGroup * grp4 + m) + c;
        x[e] = c < 3 && coord < kHeadDim ? qs[col * 132 + coord] : 0.0f;
      }
      split8(x, qh[m], ql[m]);
    }
  } else {
#pragma unroll
    for (int m = 0; m < 6; ++m) {
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int j = 8 * (m / 3) + e, c = m % 3;
        const int coord = 3 * (kTriPerGroup * grp4 + j) + c;
        x[e] = j < kTriPerGroup && coord < kHeadDim ? qs[col * 132 + coord] : 0.0f;
      }
      split8(x, qh[m], ql[m]);
    }
  }
  // QJL operands: call k, slot e of group grp4 = bit 32 grp4 + 8 k + e.
  half8 ph[QJL ? 4 : 1], pl[QJL ? 4 : 1];
  if (QJL) {
    lds_barrier();
    for (int hh = wave; hh < kMaxG; hh += kWaves) {
      float p0 = qs[hh * 132 + L] * splitmix_sign(a.kseed, kHeadDim + L);
      float p1 = qs[hh * 132 + L + 64] * splitmix_sign(a.kseed, kHeadDim + L + 64);
      wht128(p0, p1);
      wave_sync();
      // H / sqrt(d), times sqrt(pi / 2) / sqrt(d), the estimator's factor (Sec. 3.6)
      qs[hh * 132 + L] = p0 * (kInvSqrtD * kInvSqrtD * kQjlC);
      qs[hh * 132 + L + 64] = p1 * (kInvSqrtD * kInvSqrtD * kQjlC);
    }
    lds_barrier();
    // Slot map: dword m of call k (slots 2 m, 2 m + 1) stands for sign bits
    // 15 - s and 31 - s of the lane group's sign word, s = 4 k + m, so that
    // (word << s) holds them at bits 15 and 31, the fp16 sign bits.
#pragma unroll
    for (int k = 0; k < (QJL ? 4 : 1); ++k) {
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e)
        x[e] = qs[col * 132 + 32 * grp4 + ((e & 1) ? 31 : 15) - (4 * k + (e >> 1))];
      split8(x, ph[k], pl[k]);
    }
  }

  // ---- main loop: wave w takes blocks w, w+4, ... of the split
  floatx4 o[3][3];                                   // value tiles (grp, c)
#pragma unroll
  for (int i = 0; i < 3; ++i)
#pragma unroll
    for (int c = 0; c < 3; ++c) o[i][c] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
  // group codec: tile c holds columns 16 c .. 16 c + 15 (one group), and
  // zacc[j] the running sum of 64 p z of group j over this lane's tokens
  floatx4 og[8];
  float zacc[GR::G];
#pragma unroll
  for (int c = 0; c < 8; ++c) og[c] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int j = 0; j < GR::G; ++j) zacc[j] = 0.0f;
  uint32_t* vrec = reinterpret_cast<uint32_t*>(qbuf) + wave * (kIdxRows * kIdxRow / 2);
  float m_run = -INFINITY, l_run = 0.0f;            // of head `col`
  uint16_t* vidx = reinterpret_cast<uint16_t*>(qbuf) + wave * (kIdxRows * kIdxRow);
  // value-side rows of this lane's triplets 16 i + col (lanes past the last
  // triplet read a copy of it: finite values in columns never written out)
  int vrow[3];
#pragma unroll
  for (int i = 0; i < 3; ++i) vrow[i] = min(16 * i + col, kNTri - 1) * kIdxRow + 4 * grp4;
  lds_barrier();                 // every wave is done with qs before it holds indices

  const int len = max(0, min(len_raw, min(a.max_len, a.capacity)));
  // uniform: the loop and its prefetch test become scalar branches
  const int t_end = __builtin_amdgcn_readfirstlane(min(len, t_begin + a.split_len));
  // The step's (P, n) for the merge launch: P as stored (within the
  // capacity), so that the ring slots and the eviction follow the sequence's
  // state even where P exceeds max_len and the scan stops short of it.
  if (a.step && split == 0 && g == 0 && tid == 0)
    a.snap[b] = make_int2(max(0, min(len_raw, a.capacity)), max(0, min(win_raw, a.window - 1)));

  // fp16 sign bits and the fp16 pair (1, 1), in registers for and_or
  const uint32_t sgn_mask = QJL ? vreg(0x80008000u) : 0u, one_pair = QJL ? vreg(0x3C003C00u) : 0u;
  if (QJL && t0 < t_end) {                                   // (registers are short)
    load_block(blk, a, plane, t0, L);
    load_gv(blk, a, plane, t0, L);
  }
  for (; t0 < t_end; t0 += kWaves * kBlock) {
    // -- value-side triplet fields, code | rho index << 2 b_dir (the entry of
    //    a pre-split table), into this wavefront's rows (the previous block's
    //    reads of them ended at the wave_sync closing its iteration)
    if constexpr (!VG) {
      using BW = BlockWords<BD, BN, QJL, VG>;
      const int h = L >> 5, tk = L & 31;
      const uint32_t ish = (kValTri * BT * h) & 31;
      uint32_t ri[BW::KVI];
#pragma unroll
      for (int w = 0; w < BW::KVI; ++w)
        ri[w] = __builtin_amdgcn_alignbit(w + 1 < BW::KVI ? blk.vi[w + 1] : 0u, blk.vi[w], ish);
      uint16_t* row = vidx + kValTri * h * kIdxRow + tk;
#pragma unroll
      for (int j = 0; j < kValTri; ++j) row[j * kIdxRow] = (uint16_t)field<BT>(ri, j * BT);
    }
    else {
      // the group records of the block's 32 tokens as rows of 32 words:
      // code words as they are, each scale word as two rows of fp16 scales
      // (exact: every E4M3 value is an fp16 value), zero-point words as they
      // are.  Row r, token tk at vrec[32 r + tk].
      using BW = BlockWords<BD, BN, QJL, VG>;
      const int h = L >> 5, tk = L & 31;
#pragma unroll
      for (int k = 0; k < BW::KVI; ++k) {
        const int w = 2 * k + h;
        const uint32_t x = blk.vi[k];
        if (w >= GR::W) continue;
        if (w >= GR::WC && w < GR::WC + GR::G / 4) {
          const int r = GR::WC + 2 * (w - GR::WC);
          const fp16x2 lo = {(__fp16)e4m3_value(x & 0xffu), (__fp16)e4m3_value((x >> 8) & 0xffu)};
          const fp16x2 hi = {(__fp16)e4m3_value((x >> 16) & 0xffu), (__fp16)e4m3_value(x >> 24)};
          vrec[32 * r + tk] = pk(lo);
          vrec[32 * (r + 1) + tk] = pk(hi);
        } else {
          vrec[32 * (w < GR::WC ? w : w + GR::G / 4) + tk] = x;
        }
      }
    }
    // -- scores, two 16-token tiles
    floatx4 sc[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      // shift the group's window so that its triplet j starts at bit j B_tri
      using BW = BlockWords<BD, BN, QJL, VG>;
      const uint32_t ish = (kTriPerGroup * BT * grp4) & 31;
      uint32_t iw[BW::KWI];
#pragma unroll
      for (int w = 0; w < BW::KWI; ++w)
        iw[w] = __builtin_amdgcn_alignbit(w + 1 < BW::KWI ? blk.iw[kt][w + 1] : 0u, blk.iw[kt][w], ish);
      floatx4 acc = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
      if constexpr (PRE) {
#pragma unroll
        for (int m = 0; m < kTriPerGroup; ++m) {
          // triplet m of the group: its field is the entry index
          // rho K^2 + code pair, and the entry {hx|hy, hz|0, lx|ly, lz|0},
          // one 16-byte read (random gathers conflict least in wide reads),
          // is the A operand as it stands
          const half8 A = __builtin_bit_cast(half8, tabk_l[field<BT>(iw, m * BT) * kCopies]);
          acc = mfma(A, ql[m], acc);
          acc = mfma(A, qh[m], acc);
        }
      } else {
#pragma unroll
        for (int gi = 0; gi < 2; ++gi) {
          half8 ah[3], al[3];
          float ux[8], uy[8], uz[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int j = 8 * gi + e;
            if (j >= kTriPerGroup) {
              ux[e] = uy[e] = uz[e] = 0.0f;
              continue;
            }
            const uint32_t f = field<BT>(iw, j * BT);
            const uint4 n = tabk[f & (KK - 1)];
            const float rho = crk[f >> FWD];
            ux[e] = rho * __uint_as_float(n.x);
            uy[e] = rho * __uint_as_float(n.y);
            uz[e] = rho * __uint_as_float(n.z);
          }
          split8(ux, ah[0], al[0]);
          split8(uy, ah[1], al[1]);
          split8(uz, ah[2], al[2]);
#pragma unroll
          for (int c = 0; c < 3; ++c) acc = mfma3(ah[c], al[c], qh[3 * gi + c], ql[3 * gi + c], acc);
        }
      }
      // this lane's 4 tokens: t0 + 16 kt + 4 grp4 + r, head col; scores in
      // log2 units (the queries carry the softmax scale and log2 e)
      const float gka[4] = {blk.gk[kt].x, blk.gk[kt].y, blk.gk[kt].z, blk.gk[kt].w};
      float s4[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) s4[r] = acc[r] * (1.0f / kUScale);
      if (QJL) {
        const uint32_t sw = blk.sw[kt];
        floatx4 qa = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          // sigma = -1 where the bit is set: fp16 +-1 = 0x3C00 | bit << 15,
          // the two bits of dword m at 15 and 31 after the shift (slot map)
          u32x4 sg;
#pragma unroll
          for (int m = 0; m < 4; ++m) sg[m] = and_or(sw << (4 * k + m), sgn_mask, one_pair);
          const half8 sgh = __builtin_bit_cast(half8, sg);
          qa = mfma(sgh, pl[k], qa);
          qa = mfma(sgh, ph[k], qa);
        }
        const uint32_t gr2[2] = {blk.gr[kt].x, blk.gr[kt].y};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const uint16_t h = (uint16_t)(gr2[r >> 1] >> (16 * (r & 1)));
          s4[r] = fmaf((float)__builtin_bit_cast(_Float16, h), qa[r], s4[r]);
        }
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) sc[kt][r] = s4[r] * gka[r];
      if (t0 + kBlock > t_end) {          // the split's ragged last block (uniform)
        const int tb = t0 + 16 * kt + 4 * grp4;
#pragma unroll
        for (int r = 0; r < 4; ++r) sc[kt][r] = tb + r < t_end ? sc[kt][r] : -INFINITY;
      }
    }
    // -- the key words are consumed: the next block's loads go out now and
    //    land while this block's softmax and values are computed (the value
    //    norms once the softmax has read them; with QJL the registers are
    //    short: the loads go out after the values)
    //    Past the end of the split the current block is requested again (it
    //    is in cache): unconditional loads write the block's registers in
    //    place, where loads under a branch leave copies at the loop's end
    //    that wait for every outstanding load.
    const int t_next = t0 + kWaves * kBlock < t_end ? t0 + kWaves * kBlock : t0;
    if (!QJL) load_block(blk, a, plane, t_next, L);
    // -- online softmax over the 32 tokens, head col (Sec. 3.6 / App. A)
    // The value-side weight p gamma_v enters the MFMA as an fp16 hi/lo pair,
    // so it must stay below 2^16.  A token whose value norm has fp32
    // exponent byte b3 = bits >> 24 above kNormByte (gamma_v >= 128) takes
    // part in the running maximum with its (log2) score raised by
    // 2 (b3 - kNormByte), which caps p gamma_v below 2^15 for any
    // finite norm; smaller norms (b3 <= kNormByte, gamma_v < 128) leave the
    // score as it is.  The merges only need every partial's sums to share
    // the units exp(-m) of its maximum, which holds for any such shift.
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      const float gvn[4] = {blk.gv[kt].x, blk.gv[kt].y, blk.gv[kt].z, blk.gv[kt].w};
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float t = sc[kt][r];
        if constexpr (VG == 0) {
          const float b3 = (float)(__float_as_uint(gvn[r]) >> 24);
          t = fmaf(fmaxf(b3, kNormByte), 2.0f, t);
        }
        mx = fmaxf(mx, t);
      }
    }
    mx = rows_max(mx);
    if constexpr (VG == 0) mx -= 2.0f * kNormByte;
    // Lazy running maximum: a head moves its maximum (and rescales its sums)
    // only when a (raised) score exceeds it by more than kLazy, so that most
    // blocks skip the rescale; p stays below 2^kLazy = 256, p gamma_v below
    // 2^15 (or 64 p below 2^14 with group values), inside fp16, and the
    // merges cancel the shift exactly.
    const bool up = mx > m_run + kLazy;
    const float m_new = up ? mx : m_run;
    const float alpha = up ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;
    float pw[8], psum = 0.0f;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      // group codec: the weights carry the exact factor 64 of the frame
      const float gva[4] = {VG ? kUScale : blk.gv[kt].x, VG ? kUScale : blk.gv[kt].y,
                            VG ? kUScale : blk.gv[kt].z, VG ? kUScale : blk.gv[kt].w};
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        // m_new is finite here (every block holds a valid token): a masked
        // score gives exp2(-inf) = 0
        const float p = __builtin_amdgcn_exp2f(sc[kt][r] - m_new);
        psum += p;
        pw[4 * kt + r] = p * gva[r];
      }
    }
    if (!QJL) {
      // the weights are computed: the current norms are dead.  The empty asm
      // keeps the scheduler from hoisting the next norms' load above them.
      int tg = t_next;
      asm volatile("" : "+s"(tg) : "v"(pw[0]), "v"(pw[1]), "v"(pw[2]), "v"(pw[3]), "v"(pw[4]),
                   "v"(pw[5]), "v"(pw[6]), "v"(pw[7]));
      load_gv(blk, a, plane, tg, L);
    }
    psum = rows_sum(psum);
    l_run = l_run * alpha + psum;
    m_run = m_new;
    half8 pah, pal;
    split8(pw, pah, pal);
    // rescale O rows (heads 4 grp4 + r) unless no running maximum moved
    if (__ballot(alpha != 1.0f)) {
      float al[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) al[r] = __shfl(alpha, 4 * grp4 + r, 64);
      if constexpr (VG != 0) {
#pragma unroll
        for (int c = 0; c < 8; ++c)
#pragma unroll
          for (int r = 0; r < 4; ++r) og[c][r] *= al[r];
#pragma unroll
        for (int j = 0; j < GR::G; ++j) zacc[j] *= alpha;      // this lane's head: col
      } else {
#pragma unroll
        for (int i = 0; i < 3; ++i)
#pragma unroll
          for (int c = 0; c < 3; ++c)
#pragma unroll
            for (int r = 0; r < 4; ++r) o[i][c][r] *= al[r];
      }
    }
    // -- values: triplet 16 grp + col for this lane group's 8 tokens
    wave_sync();
    if constexpr (VG != 0) {
      // group codec.  Slot e of this lane group is token
      // tok(e) = 16 (e / 4) + 4 grp4 + e % 4 of the block (the score layout).
      // Tile c: B[e][col] = Delta code of column 16 c + col, exact in fp16
      // (an E4M3 scale times an integer below 16 has at most 7 significant
      // bits), so the products against the hi/lo weights are exact in the
      // fp32 accumulation; the zero-point adds sum_e 64 p_e z_e per group.
      constexpr int VB = BD - 1, kMask = (1 << VB) - 1;
      constexpr int kTilesPerGroup = VG / 16;
      const uint32_t* rq0 = vrec + 4 * grp4;                 // tokens 4 grp4 + (0..3)
#pragma unroll
      for (int j = 0; j < GR::G; ++j) {
        // fp16 scales (row WC + j / 2, half j % 2) and zero-points
        // (row WC + G / 2 + j / 2, half j % 2) of the 8 slots
        const uint4 d0 = *reinterpret_cast<const uint4*>(rq0 + 32 * (GR::WC + j / 2));
        const uint4 d1 = *reinterpret_cast<const uint4*>(rq0 + 32 * (GR::WC + j / 2) + 16);
        const uint4 z0 = *reinterpret_cast<const uint4*>(rq0 + 32 * (GR::WC + GR::G / 2 + j / 2));
        const uint4 z1 = *reinterpret_cast<const uint4*>(rq0 + 32 * (GR::WC + GR::G / 2 + j / 2) + 16);
        const uint32_t dw[8] = {d0.x, d0.y, d0.z, d0.w, d1.x, d1.y, d1.z, d1.w};
        const uint32_t zw[8] = {z0.x, z0.y, z0.z, z0.w, z1.x, z1.y, z1.z, z1.w};
        float zs = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float z = __uint_as_float(j & 1 ? (zw[e] & 0xffff0000u) : (zw[e] << 16));
          zs = fmaf(pw[e], z, zs);
        }
        zacc[j] += zs;
        fp16x2 dp[4];
#pragma unroll
        for (int m = 0; m < 4; ++m)
          dp[m] = __builtin_bit_cast(fp16x2, j & 1 ? pair_hi(dw[2 * m], dw[2 * m + 1])
                                                   : pair_lo(dw[2 * m], dw[2 * m + 1]));
#pragma unroll
        for (int cc = 0; cc < kTilesPerGroup; ++cc) {
          const int c = j * kTilesPerGroup + cc;
          // the code of column 16 c + col starts at bit pos of the record
          const int pos = (16 * c + col) * VB, wr = pos >> 5, sh = pos & 31;
          const uint4 a0 = *reinterpret_cast<const uint4*>(rq0 + 32 * wr);
          const uint4 a1 = *reinterpret_cast<const uint4*>(rq0 + 32 * wr + 16);
          uint32_t cw[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
          if constexpr ((16 * VB) % 32 != 0) {
            // 3-bit codes cross word boundaries: funnel in the next row
            const uint4 b0 = *reinterpret_cast<const uint4*>(rq0 + 32 * (wr + 1));
            const uint4 b1 = *reinterpret_cast<const uint4*>(rq0 + 32 * (wr + 1) + 16);
            const uint32_t nw[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
#pragma unroll
            for (int e = 0; e < 8; ++e) cw[e] = __builtin_amdgcn_alignbit(nw[e], cw[e], sh);
          } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) cw[e] >>= sh;
          }
          u32x4 bq;
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            // 1024 + code as fp16 (0x6400 | code), less 1024, times Delta: exact
            const uint32_t x = (cw[2 * m] & kMask) | ((cw[2 * m + 1] & kMask) << 16) | 0x64006400u;
            const fp16x2 q = __builtin_bit_cast(fp16x2, x) - fp16x2{(__fp16)1024.0f, (__fp16)1024.0f};
            bq[m] = pk(q * dp[m]);
          }
          const half8 B = __builtin_bit_cast(half8, bq);
          og[c] = mfma(pal, B, og[c]);
          og[c] = mfma(pah, B, og[c]);
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < 3; ++i) {
        // with QJL the registers are short: one value tile at a time
        if (QJL) __builtin_amdgcn_sched_barrier(0);
        // indices of tokens 4 grp4 + (0..3) and 16 + 4 grp4 + (0..3): slots e
        const uint2 p0 = *reinterpret_cast<const uint2*>(vidx + vrow[i]);
        const uint2 p1 = *reinterpret_cast<const uint2*>(vidx + vrow[i] + 16);
        const uint32_t pw2[4] = {p0.x, p0.y, p1.x, p1.y};
        half8 bh[3], bl[3];
        if (PRE) {
          uint4 E[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) E[e] = tabv_l[((pw2[e >> 1] >> (16 * (e & 1))) & 0xffffu) * kCopies];
          operands_pre(E, bh, bl);
        } else {
          float vx[8], vy[8], vz[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const uint32_t idx = (pw2[e >> 1] >> (16 * (e & 1))) & 0xffffu;
            const uint4 n = tabv[idx & (KK - 1)];
            const float rho = crv[idx >> FWD];
            vx[e] = rho * __uint_as_float(n.x);
            vy[e] = rho * __uint_as_float(n.y);
            vz[e] = rho * __uint_as_float(n.z);
          }
          split8(vx, bh[0], bl[0]);
          split8(vy, bh[1], bl[1]);
          split8(vz, bh[2], bl[2]);
        }
#pragma unroll
        for (int c = 0; c < 3; ++c) o[i][c] = mfma3(pah, pal, bh[c], bl[c], o[i][c]);
      }
    }
    if (QJL) {
      load_block(blk, a, plane, t_next, L);
      load_gv(blk, a, plane, t_next, L);
    }
    wave_sync();
  }

  // ---- merge the waves: partial (m, l, O) of this split.  The tables are
  // dead now; their LDS holds the per-wave value sums.
  lds_barrier();
  if (grp4 == 0 && col < G) {
    red_ml[(wave * kMaxG + col) * 2] = m_run;
    red_ml[(wave * kMaxG + col) * 2 + 1] = l_run;
  }
  if constexpr (VG != 0) {
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        red_o[(wave * kMaxG + 4 * grp4 + r) * kHeadDim + 16 * c + col] = og[c][r];
    // the zero-point sums of head col: its four lane groups' tokens
#pragma unroll
    for (int j = 0; j < GR::G; ++j) {
      const float z = rows_sum(zacc[j]);
      if (grp4 == 0 && col < G) red_z[(wave * kMaxG + col) * GR::G + j] = z;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 3; ++i)
#pragma unroll
      for (int c = 0; c < 3; ++c) {
        const int coord = 3 * (16 * i + col) + c;
        if (coord < kHeadDim) {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            red_o[(wave * kMaxG + 4 * grp4 + r) * kHeadDim + coord] = o[i][c][r];
        }
      }
  }
  lds_barrier();
  for (int e = tid; e < G * kHeadDim; e += kThreads) {
    const int h = e >> 7, c = e & 127;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, red_ml[(w * kMaxG + h) * 2]);
    float Lsum = 0.0f, A = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float mw = red_ml[(w * kMaxG + h) * 2];
      const float f = mw == -INFINITY ? 0.0f : exp2f(mw - M);
      Lsum += f * red_ml[(w * kMaxG + h) * 2 + 1];
      const float zt = VG ? red_z[(w * kMaxG + h) * GR::G + c / (VG ? VG : 1)] : 0.0f;
      A += f * (red_o[(w * kMaxG + h) * kHeadDim + c] + zt);
    }
    const size_t row = ((size_t)b * a.Hq + (size_t)g * G + h) * a.n_part + split;
    a.ws_acc[row * kHeadDim + c] = A;
    if (c == 0) a.ws_ml[row] = make_float2(M, Lsum);
  }
}

// Merges the partials of one (batch, query head) by their log-sum-exp and
// applies R_v^T = diag(s_v) H / sqrt(d).  Eight wavefronts take 16
// consecutive partials each per round, every load of the round in flight at
// once, with a running maximum (an online rescale) so that no pass over the
// maxima has to come first; `fold` may then add more to a wavefront's
// running (M, l, acc) (rotated frame, x64); the wavefronts meet in LDS in a
// fixed order, so the result does not depend on scheduling.
constexpr int kMergeWaves = 8;
constexpr int kMergeU = 16;

template <class Fold>
__device__ inline void merge_head(const float2* __restrict__ ws_ml, const float* __restrict__ ws_acc,
                                  int n_part, int Hq, uint64_t vseed, float* __restrict__ out,
                                  int head, int b, Fold fold) {
  __shared__ float part[kMergeWaves][2 * 64 + 2];
  const int tid = threadIdx.x, L = tid & 63, wave = tid >> 6;
  const size_t row0 = ((size_t)b * Hq + head) * n_part;
  float M = -INFINITY, Lsum = 0.0f, a0 = 0.0f, a1 = 0.0f;
  for (int s0 = wave * kMergeU; s0 < n_part; s0 += kMergeWaves * kMergeU) {
    float2 ml[kMergeU];
    float x0[kMergeU], x1[kMergeU];
#pragma unroll
    for (int u = 0; u < kMergeU; ++u) {
      const size_t r = row0 + min(s0 + u, n_part - 1);
      ml[u] = ws_ml[r];
      x0[u] = ws_acc[r * kHeadDim + L];
      x1[u] = ws_acc[r * kHeadDim + L + 64];
    }
    float m_new = M;
#pragma unroll
    for (int u = 0; u < kMergeU; ++u)
      if (s0 + u < n_part) m_new = fmaxf(m_new, ml[u].x);
    if (m_new != -INFINITY) {            // the same in every lane
      const float f0 = M == -INFINITY ? 0.0f : exp2f(M - m_new);
      Lsum *= f0;
      a0 *= f0;
      a1 *= f0;
#pragma unroll
      for (int u = 0; u < kMergeU; ++u) {
        const bool in = s0 + u < n_part && ml[u].x != -INFINITY;
        const float f = in ? exp2f(ml[u].x - m_new) : 0.0f;
        Lsum = fmaf(f, ml[u].y, Lsum);
        a0 = fmaf(f, x0[u], a0);
        a1 = fmaf(f, x1[u], a1);
      }
      M = m_new;
    }
  }
  fold(wave, L, M, Lsum, a0, a1);
  part[wave][L] = a0;
  part[wave][64 + L] = a1;
  if (L == 0) {
    part[wave][128] = M;
    part[wave][129] = Lsum;
  }
  __syncthreads();
  if (wave != 0) return;
  float Mt = -INFINITY;
#pragma unroll
  for (int w = 0; w < kMergeWaves; ++w) Mt = fmaxf(Mt, part[w][128]);
  float t0 = 0.0f, t1 = 0.0f, tl = 0.0f;
  if (Mt != -INFINITY) {
#pragma unroll
    for (int w = 0; w < kMergeWaves; ++w) {
      const float mw = part[w][128];
      const float f = mw == -INFINITY ? 0.0f : exp2f(mw - Mt);
      t0 = fmaf(f, part[w][L], t0);
      t1 = fmaf(f, part[w][64 + L], t1);
      tl = fmaf(f, part[w][129], tl);
    }
  }
  const float inv = tl > 0.0f ? 1.0f / (tl * kUScale) : 0.0f;
  t0 *= inv;
  t1 *= inv;
  wht128(t0, t1);
  const size_t o = ((size_t)b * Hq + head) * kHeadDim;
  out[o + L] = t0 * kInvSqrtD * splitmix_sign(vseed, L);
  out[o + L + 64] = t1 * kInvSqrtD * splitmix_sign(vseed, L + 64);
}

__global__ __launch_bounds__(kMergeWaves * 64) void merge_kernel(const float2* __restrict__ ws_ml,
                                                                 const float* __restrict__ ws_acc,
                                                                 int n_part, int Hq,
                                                                 uint64_t vseed,
                                                                 float* __restrict__ out) {
  merge_head(ws_ml, ws_acc, n_part, Hq, vseed, out, blockIdx.x, blockIdx.y,
             [](int, int, float&, float&, float&, float&) {});
}

// The arguments of a step's merge launch.
struct StepArgs {
  const int2* snap;                    // (P_b, n_b) as the scan read them
  int* packed_lens;
  int* win_lens;
  int window, capacity, Hkv, G;
  const void* q;
  int q_bf16;
  float scale;
  const uint16_t *k_new, *v_new;       // [B][Hkv][128] bf16
  uint16_t *k_win, *v_win;             // rings [B][Hkv][window][128] bf16
  Codebook kcb, vcb;
  int shared;                          // K and V codebook values agree
  uint64_t kseed, vseed;
  int k_rounding, v_rounding, k_qjl;
  int v_group;                         // 0, or the group size of the group value codec
  uint32_t *k_idx, *k_qjl_bits, *v_idx;   // the caches, written at slot P_b
  float *k_gamma, *v_gamma;
  uint16_t* k_gamma_r;
};

// One wavefront encodes the bf16 vector x[128] with the group-wise value
// codec into token t of `plane` (the arithmetic of the lane-per-token
// encoder, octo_encode): u = H diag(s) x / sqrt(d) with lane l holding
// coordinates l and l + 64; a group of GS coordinates is GS consecutive
// lanes, so its range is an xor-shuffle reduction (exact in any order); the
// record's words are then assembled from the codes in `scr` (at least
// 128 + 2 * 128 / GS words) by lanes w < W.
template <int VB, int GS>
__device__ void encode_group_one(const uint16_t* x, uint64_t seed, uint32_t* idx, size_t plane,
                                 int capacity, int t, uint32_t* scr) {
  constexpr int G = kHeadDim / GS, WC = VB * kHeadDim / 32, W = group_record_words(VB, GS);
  constexpr float kLevels = (float)((1 << VB) - 1);
  const int L = threadIdx.x & 63;
  float u[2] = {bf16_to_f32(x[L]) * splitmix_sign(seed, L),
                bf16_to_f32(x[L + 64]) * splitmix_sign(seed, L + 64)};
  wht128(u[0], u[1]);
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const float v = u[k] * kInvSqrtD;
    float mn = v, mx = v;
#pragma unroll
    for (int m = 1; m < GS; m <<= 1) {
      mn = fminf(mn, __shfl_xor(mn, m, 64));
      mx = fmaxf(mx, __shfl_xor(mx, m, 64));
    }
    mn += 0.0f;                          // a zero minimum is stored as +0
    const uint32_t s8 = e4m3_rne((mx - mn) / kLevels);
    const float dh = e4m3_value(s8);
    const uint32_t z16 = bf16_rne(mn);
    const float zh = __uint_as_float(z16 << 16);
    const float qf = fminf(fmaxf(rintf((v - zh) / dh), 0.0f), kLevels);
    const int c = L + 64 * k;
    scr[c] = dh > 0.0f ? (uint32_t)qf : 0u;
    if (c % GS == 0) {
      scr[kHeadDim + c / GS] = s8;
      scr[kHeadDim + G + c / GS] = z16;
    }
  }
  wave_sync();
  if (L < W) {
    uint32_t word = 0u;
    if (L < WC) {
      // codes whose bits meet [32 L, 32 L + 32)
      for (int c = (32 * L) / VB; c < kHeadDim && c * VB < 32 * L + 32; ++c) {
        const int sh = c * VB - 32 * L;
        word |= sh >= 0 ? scr[c] << sh : scr[c] >> -sh;
      }
    } else if (L < WC + G / 4) {
      const int j = 4 * (L - WC);
#pragma unroll
      for (int k = 0; k < 4; ++k) word |= scr[kHeadDim + j + k] << (8 * k);
    } else {
      const int j = 2 * (L - WC - G / 4);
      word = scr[kHeadDim + G + j] | (scr[kHeadDim + G + j + 1] << 16);
    }
    idx[tile_word(plane, capacity, t, L, W)] = word;
  }
}

// The append workgroup of sequence b: the new tokens to their ring slots,
// the tokens leaving full rings encoded into packed slot P (one wavefront per
// vector; the ring row, or the new row when the window is one token), and
// the lengths.
template <int BD, int BN>
__device__ void append_block(const StepArgs& a, int b) {
  constexpr int K = 1 << BD, R = 1 << BN, KP = K + 2;
  __shared__ float cx_k[K], cx_v[K], cr_k[R], cr_v[R];
  __shared__ floatx4 lut[2][KP * KP];
  __shared__ float midp[2][K + 1], mid_rho[2][R > 1 ? R - 1 : 1];
  __shared__ float scratch[kMergeWaves][192];
  constexpr int kThreads = kMergeWaves * 64;
  const int tid = threadIdx.x, L = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int W = a.window;
  const int P = a.snap[b].x, n = a.snap[b].y, t = P + n;
  for (int e = tid; e < a.Hkv * 2 * kHeadDim; e += kThreads) {
    const int gq = e / (2 * kHeadDim), r = e % (2 * kHeadDim), c = r & (kHeadDim - 1);
    const size_t plane = (size_t)b * a.Hkv + gq;
    uint16_t* ring = r < kHeadDim ? a.k_win : a.v_win;
    const uint16_t* src = r < kHeadDim ? a.k_new : a.v_new;
    ring[(plane * W + t % W) * kHeadDim + c] = src[plane * kHeadDim + c];
  }
  const bool evict = n + 1 == W && P < a.capacity;
  if (evict) {
    // the codebooks at constant indices (scalar loads of the kernel arguments)
    float xk = 0.0f, xv = 0.0f, rk = 0.0f, rv = 0.0f;
#pragma unroll
    for (int i = 0; i < K; ++i) {
      xk = L == i ? a.kcb.xi[i] : xk;
      xv = L == i ? a.vcb.xi[i] : xv;
    }
#pragma unroll
    for (int i = 0; i < R; ++i) {
      rk = L == i ? a.kcb.rho[i] : rk;
      rv = L == i ? a.vcb.rho[i] : rv;
    }
    if (tid < K) {
      cx_k[tid] = xk;
      cx_v[tid] = xv;
    }
    if (tid < R) {
      cr_k[tid] = rk;
      cr_v[tid] = rv;
    }
    __syncthreads();
    encoder_tables<BD, BN>(cx_k, cr_k, lut[0], midp[0], mid_rho[0], tid, kThreads);
    const int vt = a.shared ? 0 : 1;
    if (!a.shared) encoder_tables<BD, BN>(cx_v, cr_v, lut[1], midp[1], mid_rho[1], tid, kThreads);
    __syncthreads();
    for (int item = wave; item < 2 * a.Hkv; item += kMergeWaves) {
      const int gq = item >> 1;
      const bool v = item & 1;
      const size_t plane = (size_t)b * a.Hkv + gq;
      const uint16_t* src = n == 0 ? (v ? a.v_new : a.k_new) + plane * kHeadDim
                                   : (v ? a.v_win : a.k_win) + (plane * W + P % W) * kHeadDim;
      float* u = scratch[wave];
      uint32_t* fld = reinterpret_cast<uint32_t*>(u + 132);
      if (v && a.v_group) {
        if constexpr (BD == BN + 2) {       // the group codec has b = b_dir - 1 bits here
          uint32_t* scr = reinterpret_cast<uint32_t*>(u);
          if (a.v_group == 16)
            encode_group_one<BD - 1, 16>(src, a.vseed, a.v_idx, plane, a.capacity, P, scr);
          else
            encode_group_one<BD - 1, 32>(src, a.vseed, a.v_idx, plane, a.capacity, P, scr);
        }
      } else if (v)
        encode_one<BD, BN>(src, lut[vt], midp[vt], mid_rho[vt], cr_v, a.vseed, a.v_rounding,
                           false, a.v_idx, a.v_gamma, nullptr, nullptr, plane, a.capacity, P,
                           u, fld);
      else
        encode_one<BD, BN>(src, lut[0], midp[0], mid_rho[0], cr_k, a.kseed, a.k_rounding,
                           a.k_qjl != 0, a.k_idx, a.k_gamma, a.k_qjl_bits, a.k_gamma_r, plane,
                           a.capacity, P, u, fld);
      wave_sync();                       // the scratch is reused by the next item
    }
  }
  if (tid == 0) {
    if (evict) a.packed_lens[b] = P + 1;
    a.win_lens[b] = n + 1 < W ? n + 1 : n;
  }
}

// A step's merge: blocks (head, b) merge the scan's partials and fold in the
// native rows of tokens P .. P + n (the last one the new token), wavefront w
// taking tokens j = w, w + 8, ... with its own online softmax, four tokens'
// loads in flight at a time; its sum goes into the value frame (x64) as the
// scan's are.  Block (Hq, b) is the append workgroup.
constexpr int kFoldChunk = 4;
template <int BD, int BN>
__global__ __launch_bounds__(kMergeWaves * 64) void step_merge_kernel(
    const float2* __restrict__ ws_ml, const float* __restrict__ ws_acc, int n_part, int Hq,
    float* __restrict__ out, StepArgs a) {
  const int b = blockIdx.y;
  if ((int)blockIdx.x == Hq) {
    append_block<BD, BN>(a, b);
    return;
  }
  const int head = blockIdx.x, g = head / a.G;
  const int W = a.window, P = a.snap[b].x, n = a.snap[b].y;
  const size_t plane = (size_t)b * a.Hkv + g;
  merge_head(ws_ml, ws_acc, n_part, Hq, a.vseed, out, head, b,
             [&](int wave, int L, float& M, float& Lsum, float& a0, float& a1) {
    const size_t qo = ((size_t)b * Hq + head) * kHeadDim;
    float q0, q1;
    if (a.q_bf16) {
      q0 = bf16_to_f32(static_cast<const uint16_t*>(a.q)[qo + L]);
      q1 = bf16_to_f32(static_cast<const uint16_t*>(a.q)[qo + L + 64]);
    } else {
      q0 = static_cast<const float*>(a.q)[qo + L];
      q1 = static_cast<const float*>(a.q)[qo + L + 64];
    }
    float wm = -INFINITY, wl = 0.0f, w0 = 0.0f, w1 = 0.0f;
    for (int j0 = wave; j0 <= n; j0 += kFoldChunk * kMergeWaves) {
      uint16_t k0[kFoldChunk], k1[kFoldChunk], v0[kFoldChunk], v1[kFoldChunk];
#pragma unroll
      for (int c = 0; c < kFoldChunk; ++c) {
        // tokens past the window read the new token's row (never used)
        const int j = min(j0 + c * kMergeWaves, n);
        const size_t row = (plane * W + (P + j) % W) * kHeadDim;
        const uint16_t* kr = j == n ? a.k_new + plane * kHeadDim : a.k_win + row;
        const uint16_t* vr = j == n ? a.v_new + plane * kHeadDim : a.v_win + row;
        k0[c] = kr[L];
        k1[c] = kr[L + 64];
        v0[c] = vr[L];
        v1[c] = vr[L + 64];
      }
#pragma unroll
      for (int c = 0; c < kFoldChunk; ++c) {
        if (j0 + c * kMergeWaves > n) break;
        const float s =
            a.scale * wave_sum(fmaf(q0, bf16_to_f32(k0[c]), q1 * bf16_to_f32(k1[c])));
        const float mn = fmaxf(wm, s);
        const float f = exp2f(wm - mn), p = exp2f(s - mn);
        wl = fmaf(wl, f, p);
        w0 = fmaf(w0, f, p * bf16_to_f32(v0[c]));
        w1 = fmaf(w1, f, p * bf16_to_f32(v1[c]));
        wm = mn;
      }
    }
    if (wm != -INFINITY) {              // the same in every lane
      // R_v v = H diag(s_v) v / sqrt(d), x64 like the scan's sums
      float x0 = w0 * splitmix_sign(a.vseed, L), x1 = w1 * splitmix_sign(a.vseed, L + 64);
      wht128(x0, x1);
      const float mn = fmaxf(M, wm);
      const float fa = M == -INFINITY ? 0.0f : exp2f(M - mn), fb = exp2f(wm - mn);
      Lsum = fmaf(Lsum, fa, wl * fb);
      a0 = fmaf(a0, fa, x0 * (kInvSqrtD * kUScale) * fb);
      a1 = fmaf(a1, fa, x1 * (kInvSqrtD * kUScale) * fb);
      M = mn;
    }
  });
}

struct Plan {
  int n_split, split_len;
  size_t ml_bytes, acc_bytes, snap_bytes, total;
};

// Splits of `nw`-wave workgroups: about eight waves per CU in all, each
// split a multiple of nw 32-token blocks; a step also keeps each sequence's
// (P, n) after the partials.
Plan make_plan(int B, int Hq, int Hkv, int max_len, int nw, bool step) {
  Plan p;
  const int units = B * Hkv;
  const int target_blocks = 256 * (8 / nw);
  const int quantum = nw * kBlock;
  const int per_unit = max(1, target_blocks / max(1, units));
  int sl = (max(max_len, 1) + per_unit - 1) / per_unit;
  sl = (sl + quantum - 1) / quantum * quantum;
  p.split_len = max(sl, quantum);
  p.n_split = max(1, (max_len + p.split_len - 1) / p.split_len);
  const size_t rows = (size_t)B * Hq * p.n_split;
  p.ml_bytes = (rows * sizeof(float2) + 255) / 256 * 256;
  p.acc_bytes = rows * kHeadDim * sizeof(float);
  p.snap_bytes = step ? ((size_t)B * sizeof(int2) + 255) / 256 * 256 : 0;
  p.total = p.ml_bytes + p.acc_bytes + p.snap_bytes;
  return p;
}

// Big tables (more than kMaxSmallPre entries) are pre-split only when K and
// V share their codebooks (one table fills the CU's LDS); otherwise fp32.
bool big_split(int b_dir, int b_nrm) { return (1 << (2 * b_dir + b_nrm)) > kMaxSmallPre; }
int waves_for(int b_dir, int b_nrm, bool shared) {
  return big_split(b_dir, b_nrm) && shared ? kWavesBig : kWavesSmall;
}

template <int BD, int BN, bool QJL>
void launch_q(const DecodeArgs& a, int vg, hipStream_t st) {
  dim3 grid(a.n_split, a.Hkv, a.B);
  constexpr bool big = (1 << (2 * BD + BN)) > kMaxSmallPre;
  constexpr int NW = big ? kWavesBig : kWavesSmall;
  if constexpr (BD == BN + 2) {
    // the group-wise value codec with b = b_dir - 1 bits: one (K) table
    if (vg == 16) {
      hipLaunchKernelGGL((decode_kernel<BD, BN, QJL, kPre, NW, 16>), grid, dim3(64 * NW), 0, st, a);
      return;
    }
    if (vg == 32) {
      hipLaunchKernelGGL((decode_kernel<BD, BN, QJL, kPre, NW, 32>), grid, dim3(64 * NW), 0, st, a);
      return;
    }
  }
  if constexpr (!big) {
    hipLaunchKernelGGL((decode_kernel<BD, BN, QJL, kPre, kWavesSmall>), grid, dim3(64 * kWavesSmall), 0, st, a);
  } else {
    if (a.shared_tables)
      hipLaunchKernelGGL((decode_kernel<BD, BN, QJL, kPre, kWavesBig>), grid, dim3(64 * kWavesBig), 0, st, a);
    else
      hipLaunchKernelGGL((decode_kernel<BD, BN, QJL, kFp32, kWavesSmall>), grid, dim3(64 * kWavesSmall), 0, st, a);
  }
}

template <int BD, int BN>
void launch(const DecodeArgs& a, bool qjl, int vg, hipStream_t st) {
  if (qjl)
    launch_q<BD, BN, true>(a, vg, st);
  else
    launch_q<BD, BN, false>(a, vg, st);
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
  if (kc->group) return fail(OCTO_ERR_UNSUPPORTED, "%s: keys need the OCTOPUS codec", what);
  if (vc->qjl) return fail(OCTO_ERR_UNSUPPORTED, "%s: the value codec cannot carry QJL", what);
  if (vc->group) {
    if (kc->b_dir != kc->b_nrm + 2 || vc->bits != kc->bits)
      return fail(OCTO_ERR_UNSUPPORTED,
                  "%s: a group value codec needs keys in the (b+1, b-1) split with the same b", what);
  } else if (kc->b_dir != vc->b_dir || kc->b_nrm != vc->b_nrm) {
    return fail(OCTO_ERR_UNSUPPORTED, "%s: K and V must share (b_dir, b_nrm)", what);
  }
  if (k_cache->batch != v_cache->batch || k_cache->kv_heads != v_cache->kv_heads ||
      k_cache->capacity != v_cache->capacity)
    return fail(OCTO_ERR_INVALID_ARGUMENT, "%s: K and V caches differ in shape", what);
  return OCTO_OK;
}

// Checks shared by octo_attend_decode and octo_decode_step and the
// arguments of the scan (no step fields but the snapshot's place).
static octo_status prepare(const char* what, const octo_codec_desc* k_codec,
                           const octo_codec_desc* v_codec, const octo_cache_view* k_cache,
                           const octo_cache_view* v_cache, const void* q, int32_t q_dtype,
                           int32_t num_q_heads, const int32_t* seq_lens, int32_t max_seq_len,
                           float softmax_scale, float* out, void* workspace,
                           size_t workspace_bytes, bool step, DecodeArgs* a, Codec* kc, Codec* vc) {
  octo_status s = check_kv(k_codec, v_codec, k_cache, v_cache, what, kc, vc);
  if (s != OCTO_OK) return s;
  if (q_dtype != OCTO_DTYPE_F32 && q_dtype != OCTO_DTYPE_BF16)
    return fail(OCTO_ERR_INVALID_ARGUMENT, "%s: q_dtype %d unknown", what, (int)q_dtype);
  if (!q || !seq_lens || !out)
    return fail(OCTO_ERR_INVALID_ARGUMENT, "%s: q, the lengths and out must be set", what);
  if ((uintptr_t)q % (q_dtype == OCTO_DTYPE_F32 ? 4 : 2) || ((uintptr_t)seq_lens & 3) ||
      ((uintptr_t)out & 3))
    return fail(OCTO_ERR_ALIGNMENT, "%s: q, the lengths or out misaligned", what);
  const int B = k_cache->batch, Hkv = k_cache->kv_heads;
  if (num_q_heads < 1 || num_q_heads % Hkv)
    return fail(OCTO_ERR_INVALID_ARGUMENT, "%s: %d query heads on %d KV heads", what,
                num_q_heads, Hkv);
  const int G = num_q_heads / Hkv;
  if (G > kMaxG)
    return fail(OCTO_ERR_UNSUPPORTED, "%s: %d query heads per KV head (at most %d)", what, G,
                kMaxG);
  if (max_seq_len < 0 || max_seq_len > k_cache->capacity)
    return fail(OCTO_ERR_CAPACITY, "%s: max length %d outside [0, capacity %d]", what,
                max_seq_len, k_cache->capacity);
  if (B > 65535 || Hkv > 65535 || num_q_heads > 65535)
    return fail(OCTO_ERR_UNSUPPORTED, "%s: batch and heads must be <= 65535", what);
  // a group value codec needs no table of its own: the big K table is alone
  const bool shared = vc->group || std::memcmp(&kc->cb, &vc->cb, sizeof(Codebook)) == 0;
  const Plan p =
      make_plan(B, num_q_heads, Hkv, max_seq_len, waves_for(kc->b_dir, kc->b_nrm, shared), step);
  if (!workspace || workspace_bytes < p.total)
    return fail(OCTO_ERR_WORKSPACE_TOO_SMALL, "%s: workspace %zu bytes, need %zu", what,
                workspace_bytes, p.total);
  if ((uintptr_t)workspace & 255)
    return fail(OCTO_ERR_ALIGNMENT, "%s: workspace must be 256-byte aligned", what);

  std::memset(a, 0, sizeof(*a));
  a->q = q;
  a->q_bf16 = q_dtype == OCTO_DTYPE_BF16;
  a->B = B;
  a->Hq = num_q_heads;
  a->Hkv = Hkv;
  a->G = G;
  a->seq_lens = seq_lens;
  a->max_len = max_seq_len;
  a->scale = softmax_scale > 0.0f ? softmax_scale : kInvSqrtD;
  a->kcb = kc->cb;
  a->vcb = vc->cb;
  a->shared_tables = shared;
  a->v_group = vc->group;
  a->kseed = kc->seed;
  a->vseed = vc->seed;
  a->k_idx = k_cache->idx;
  a->kqjl = k_cache->qjl;
  a->kgamma = k_cache->gamma;
  a->kgamma_r = k_cache->gamma_r;
  a->v_idx = v_cache->idx;
  a->vgamma = v_cache->gamma;          // NULL with a group value codec (unread)
  a->capacity = k_cache->capacity;
  a->n_split = p.n_split;
  a->split_len = p.split_len;
  a->n_part = p.n_split;
  char* ws = static_cast<char*>(workspace);
  a->ws_ml = reinterpret_cast<float2*>(ws);
  a->ws_acc = reinterpret_cast<float*>(ws + p.ml_bytes);
  a->snap = step ? reinterpret_cast<int2*>(ws + p.ml_bytes + p.acc_bytes) : nullptr;
  return OCTO_OK;
}

static octo_status launch_scan(const DecodeArgs& a, const Codec& kc, const char* what,
                               hipStream_t stream) {
  const int vg = a.v_group;
  switch (kc.b_dir * 10 + kc.b_nrm) {
    case 31: launch<3, 1>(a, kc.qjl, vg, stream); break;
    case 42: launch<4, 2>(a, kc.qjl, vg, stream); break;
    case 53: launch<5, 3>(a, kc.qjl, vg, stream); break;
    case 22: launch<2, 2>(a, kc.qjl, vg, stream); break;
    case 33: launch<3, 3>(a, kc.qjl, vg, stream); break;
    case 44: launch<4, 4>(a, kc.qjl, vg, stream); break;
    default: return fail(OCTO_ERR_UNSUPPORTED, "%s: configuration not compiled", what);
  }
  return check_launch(what);
}

static octo_status workspace_bytes_for(const char* what, const octo_codec_desc* k_codec,
                                       int32_t B, int32_t num_q_heads, int32_t kv_heads,
                                       int32_t max_len, bool step, size_t* bytes) {
  Codec kc;
  octo_status s = resolve_codec(k_codec, what, &kc, false);
  if (s != OCTO_OK) return s;
  if (kc.group) return fail(OCTO_ERR_UNSUPPORTED, "%s: keys need the OCTOPUS codec", what);
  if (!bytes) return fail(OCTO_ERR_INVALID_ARGUMENT, "%s: bytes is NULL", what);
  if (B < 1 || num_q_heads < 1 || kv_heads < 1 || max_len < 0)
    return fail(OCTO_ERR_INVALID_ARGUMENT, "%s: bad sizes", what);
  // the small-workgroup plan has the most splits: enough for either
  *bytes = make_plan(B, num_q_heads, kv_heads, max_len, kWavesSmall, step).total;
  return OCTO_OK;
}

extern "C" octo_status octo_decode_workspace_bytes(const octo_codec_desc* k_codec, int32_t B,
                                                   int32_t num_q_heads, int32_t kv_heads,
                                                   int32_t max_seq_len, size_t* bytes) {
  clear_error();
  return workspace_bytes_for("octo_decode_workspace_bytes", k_codec, B, num_q_heads, kv_heads,
                             max_seq_len, false, bytes);
}

static octo_status attend_decode(const char* what, const octo_codec_desc* k_codec,
                                 const octo_codec_desc* v_codec, const octo_cache_view* k_cache,
                                 const octo_cache_view* v_cache, const void* q,
                                 int32_t q_dtype, int32_t num_q_heads,
                                 const int32_t* seq_lens, int32_t max_seq_len,
                                 float softmax_scale, float* out, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream) {
  DecodeArgs a;
  Codec kc, vc;
  octo_status s = prepare(what, k_codec, v_codec, k_cache, v_cache, q, q_dtype, num_q_heads,
                          seq_lens, max_seq_len, softmax_scale, out, workspace, workspace_bytes,
                          false, &a, &kc, &vc);
  if (s != OCTO_OK) return s;
  if ((s = launch_scan(a, kc, what, stream)) != OCTO_OK) return s;
  hipLaunchKernelGGL(merge_kernel, dim3(num_q_heads, a.B), dim3(kMergeWaves * 64), 0, stream,
                     a.ws_ml, a.ws_acc, a.n_part, num_q_heads, vc.seed, out);
  return check_launch(what);
}

extern "C" octo_status octo_attend_decode(const octo_codec_desc* k_codec,
                                          const octo_codec_desc* v_codec,
                                          const octo_cache_view* k_cache,
                                          const octo_cache_view* v_cache, const void* q,
                                          int32_t q_dtype, int32_t num_q_heads,
                                          const int32_t* seq_lens, int32_t max_seq_len,
                                          float softmax_scale, float* out, void* workspace,
                                          size_t workspace_bytes, hipStream_t stream) {
  clear_error();
  return attend_decode("octo_attend_decode", k_codec, v_codec, k_cache, v_cache, q, q_dtype,
                       num_q_heads, seq_lens, max_seq_len, softmax_scale, out, workspace,
                       workspace_bytes, stream);
}

// ---------------------------------------------------------------- no-alloc variant
// octo_attend_decode_noalloc keeps the per-split partials of a call in this
// device array instead of a caller's workspace.  Each GPU the library runs on
// holds its own copy until the process ends.  In host code the array's name
// is not a device address: every host use goes through the address that
// hipGetSymbolAddress returns for the current device, looked up once per
// device and kept in g_scratch_ptr.
constexpr size_t kScratchBytes = size_t(16) << 20;
static __device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices];

// The current device's address of `scratch`, resolved on the first call on
// that device.
static octo_status scratch_address(const char* what, void** ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0)
    return fail(OCTO_ERR_HIP, "%s: no current HIP device", what);
  if (dev >= kMaxDevices)
    return fail(OCTO_ERR_UNSUPPORTED, "%s: device %d (at most %d devices)", what, dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(OCTO_ERR_HIP, "%s: hipGetSymbolAddress of the scratch array failed on device %d: %s",
                  what, dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return OCTO_OK;
}

extern "C" octo_status octo_attend_decode_noalloc(const octo_codec_desc* k_codec,
                                                  const octo_codec_desc* v_codec,
                                                  const octo_cache_view* k_cache,
                                                  const octo_cache_view* v_cache, const void* q,
                                                  int32_t q_dtype, int32_t num_q_heads,
                                                  const int32_t* seq_lens, int32_t max_seq_len,
                                                  float softmax_scale, float* out,
                                                  hipStream_t stream) {
  clear_error();
  const char* what = "octo_attend_decode_noalloc";
  // the same split plan as octo_attend_decode: its partials must fit the array
  if (!k_cache) return fail(OCTO_ERR_INVALID_ARGUMENT, "%s: k_cache is NULL", what);
  size_t need = 0;
  octo_status s = workspace_bytes_for(what, k_codec, k_cache->batch, num_q_heads,
                                      k_cache->kv_heads, max_seq_len, false, &need);
  if (s != OCTO_OK) return s;
  if (need > kScratchBytes)
    return fail(OCTO_ERR_CAPACITY,
                "%s: these shapes need %zu bytes of partials, more than the %zu-byte static "
                "scratch; use octo_attend_decode with a workspace", what, need, kScratchBytes);
  void* ptr = nullptr;
  if ((s = scratch_address(what, &ptr)) != OCTO_OK) return s;
  return attend_decode(what, k_codec, v_codec, k_cache, v_cache, q, q_dtype, num_q_heads,
                       seq_lens, max_seq_len, softmax_scale, out, ptr, kScratchBytes, stream);
}

extern "C" octo_status octo_decode_step_workspace_bytes(const octo_codec_desc* k_codec, int32_t B,
                                                        int32_t num_q_heads, int32_t kv_heads,
                                                        int32_t max_packed_len, size_t* bytes) {
  clear_error();
  return workspace_bytes_for("octo_decode_step_workspace_bytes", k_codec, B, num_q_heads,
                             kv_heads, max_packed_len, true, bytes);
}

extern "C" octo_status octo_decode_step(const octo_codec_desc* k_codec,
                                        const octo_codec_desc* v_codec,
                                        const octo_cache_view* k_cache,
                                        const octo_cache_view* v_cache, const void* q,
                                        int32_t q_dtype, int32_t num_q_heads,
                                        const uint16_t* k_new, const uint16_t* v_new,
                                        uint16_t* k_window, uint16_t* v_window, int32_t window,
                                        int32_t* packed_lens, int32_t* window_lens,
                                        int32_t max_packed_len, float softmax_scale, float* out,
                                        void* workspace, size_t workspace_bytes,
                                        hipStream_t stream) {
  clear_error();
  const char* what = "octo_decode_step";
  DecodeArgs a;
  Codec kc, vc;
  octo_status s = prepare(what, k_codec, v_codec, k_cache, v_cache, q, q_dtype, num_q_heads,
                          packed_lens, max_packed_len, softmax_scale, out, workspace,
                          workspace_bytes, true, &a, &kc, &vc);
  if (s != OCTO_OK) return s;
  if (window < 1 || window > kMaxWindow)
    return fail(OCTO_ERR_UNSUPPORTED, "%s: window %d outside [1, %d]", what, window, kMaxWindow);
  if (!k_new || !v_new || !k_window || !v_window || !window_lens)
    return fail(OCTO_ERR_INVALID_ARGUMENT, "%s: new rows, rings and window_lens must be set", what);
  if (((uintptr_t)k_new | (uintptr_t)v_new | (uintptr_t)k_window | (uintptr_t)v_window) & 15 ||
      ((uintptr_t)window_lens & 3))
    return fail(OCTO_ERR_ALIGNMENT, "%s: rows or window_lens misaligned", what);
  a.step = 1;
  a.window = window;
  a.win_lens = window_lens;
  if ((s = launch_scan(a, kc, what, stream)) != OCTO_OK) return s;
  StepArgs st;
  std::memset(&st, 0, sizeof(st));
  st.snap = a.snap;
  st.packed_lens = packed_lens;
  st.win_lens = window_lens;
  st.window = window;
  st.capacity = k_cache->capacity;
  st.Hkv = a.Hkv;
  st.G = a.G;
  st.q = q;
  st.q_bf16 = a.q_bf16;
  st.scale = a.scale * kLog2e;          // the fold's scores in log2 units, as the scan's
  st.k_new = k_new;
  st.v_new = v_new;
  st.k_win = k_window;
  st.v_win = v_window;
  st.kcb = kc.cb;
  st.vcb = vc.cb;
  st.shared = a.shared_tables;
  st.kseed = kc.seed;
  st.vseed = vc.seed;
  st.k_rounding = kc.rounding;
  st.v_rounding = vc.rounding;
  st.k_qjl = kc.qjl;
  st.v_group = vc.group;
  st.k_idx = k_cache->idx;
  st.k_qjl_bits = k_cache->qjl;
  st.k_gamma = k_cache->gamma;
  st.k_gamma_r = k_cache->gamma_r;
  st.v_idx = v_cache->idx;
  st.v_gamma = v_cache->gamma;
  const dim3 grid(num_q_heads + 1, a.B), block(kMergeWaves * 64);
#define OCTO_STEP_MERGE(BD, BN)                                                                   \
  hipLaunchKernelGGL((step_merge_kernel<BD, BN>), grid, block, 0, stream, a.ws_ml, a.ws_acc, \
                     a.n_part, num_q_heads, out, st)
  switch (kc.b_dir * 10 + kc.b_nrm) {
    case 31: OCTO_STEP_MERGE(3, 1); break;
    case 42: OCTO_STEP_MERGE(4, 2); break;
    case 53: OCTO_STEP_MERGE(5, 3); break;
    case 22: OCTO_STEP_MERGE(2, 2); break;
    case 33: OCTO_STEP_MERGE(3, 3); break;
    case 44: OCTO_STEP_MERGE(4, 4); break;
    default: return fail(OCTO_ERR_UNSUPPORTED, "%s: configuration not compiled", what);
  }
#undef OCTO_STEP_MERGE
  return check_launch(what);
}
