// octo_encode: the OCTOPUS encoder on gfx950.
//
// Each token follows the OCTOPUS paper (arXiv 2605.21226):
//   Sec. 3.1      gamma = ||x||_2 and u = R x / gamma with R = H diag(s)
//                 (the SplitMix64 signs as 128-bit wave-ballot masks);
//   Sec. 3.2      u zero-padded to 129 coordinates, 43 triplets t_i, the
//                 octahedral coordinates (xi, eta) of Eq. 5;
//   Sec. 3.5      scalar Lloyd seeds, then the local 3x3 joint rounding: the
//                 candidate direction maximizing s = t . n(xi^, eta^) and the
//                 norm centroid nearest that s (the minimizer of Eq. 12);
//                 rounding = SCALAR keeps the seeds and the centroid nearest
//                 rho = ||t||;
//   Sec. 3.6      with QJL: r = u - u^, sigma = sign(H diag(s') r) and
//                 gamma_r = fp16(||r||);
//   Sec. 3        the indices of I_dir and I_nrm as one field per triplet
//                 (xi | eta << b_dir | rho << 2 b_dir, B_tri bits).
// encode_part_kernel gives each token four lanes and forms the rotation on
// the matrix cores (see its section).  group_encode_kernel encodes the
// group-wise value codec, one lane a token with the row in 128 registers.
// In the tile-64 layout word w of 64 consecutive tokens is 256 contiguous
// bytes, so the word stores are coalesced.  LDS holds the codebooks, their
// cell boundaries and, for every code pair, the decoded unit direction
// n(xi^, eta^) with the pair's code, in a table padded by one clamped cell
// per side so that the 3x3 search is nine reads at constant offsets and two
// selects per candidate.
#include <math.h>

#include <algorithm>
#include <type_traits>

#include "octo_internal.h"

namespace octo {
namespace {

constexpr int kThreads = 256;     // tokens per workgroup, one per lane
constexpr float kInvSqrtD = 0.08838834764831845f;

struct EncodeArgs {
  const void* x;
  int64_t s0, s1, s2;             // element strides of b, h, t
  int is_bf16, vec16;             // vec16: every row starts 16-byte aligned
  int B, H, T;
  WideCodebook cb;                // C_xi, C_rho values
  uint64_t seed;
  int qjl, rounding;
  uint32_t* idx;                  // index stream, one B_tri-bit field per triplet
  float* gamma;
  uint32_t* qjl_bits;
  uint16_t* gamma_r;
  int capacity, token_offset;
  // signs of R and R' (bit k % 32 of word k / 32: s_k < 0), from the seed
  uint32_t smask[4], qmask[4];
  int tiles;                      // 16-token tiles a wavefront (multi-tile kernels)
};

// Nearest of the K sorted centroids of C_xi: the number of the K-1 cell
// boundaries below x.  `midp` holds them padded, midp[0] = -inf,
// midp[k] = (c_(k-1) + c_k) / 2, midp[K] = +inf.  The Lloyd-Max centroids on
// [-1, 1] lie close to a uniform grid; when every boundary is within one grid
// cell of the uniform one (checked per workgroup), the grid cell g of x is at
// most one index off and the two boundaries around g give the exact count.
template <int K>
__device__ inline int seed_guess(const float* midp, float x) {
  int g = (int)fmaf(x, 0.5f * K, 0.5f * K);
  g = min(max(g, 0), K - 1);
  const float dn = midp[g], up = midp[g + 1];
  const int r = g - 1 + (x > dn ? 1 : 0) + (x > up ? 1 : 0);
  return min(max(r, 0), K - 1);      // (only a NaN input could leave the range)
}

// The same count by binary search, for codebooks far from the uniform grid.
template <int K>
__device__ inline int seed_search(const float* midp, float x) {
  int idx = 0;
#pragma unroll
  for (int step = K >> 1; step > 0; step >>= 1)
    if (x > midp[idx + step]) idx += step;
  return idx;
}

// The same count for the few C_rho boundaries held in registers.
template <int R>
__device__ inline int rho_index(const float (&mid)[R > 1 ? R - 1 : 1], float x) {
  int idx = 0;
#pragma unroll
  for (int k = 0; k < R - 1; ++k) idx += x > mid[k] ? 1 : 0;
  return idx;
}

// Calls f(std::integral_constant<int, I>) for I = B .. E-1: the register
// array indices in the body stay compile-time constants however large the
// body is (a pragma unroll gives up on the 43 encoder triplets).
template <int B, int E>
struct StaticFor {
  template <class F>
  __device__ static inline void run(F&& f) {
    f(std::integral_constant<int, B>{});
    StaticFor<B + 1, E>::run(f);
  }
};
template <int E>
struct StaticFor<E, E> {
  template <class F>
  __device__ static inline void run(F&&) {}
};

// Materializes x in a register at this point.  The compiler otherwise sinks
// the rotation into the triplet loop and turns the table selects below into
// branches around partial loads.
typedef float floatx4 __attribute__((ext_vector_type(4)));
__device__ inline void pin(float& x) { asm volatile("" : "+v"(x)); }
__device__ inline void pin(floatx4& x) { asm volatile("" : "+v"(x)); }

// Unnormalized Walsh-Hadamard transform of 128 registers (Sylvester order).
// One stage at a time: interleaving the stages only lengthens live ranges.
__device__ inline void wht128_regs(float (&v)[128]) {
#pragma unroll
  for (int h = 1; h < 128; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 128; ++i)
      if (!(i & h)) {
        const float p = v[i], q = v[i + h];
        v[i] = p + q;
        v[i + h] = p - q;
      }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Flips the sign of v[j] where bit j of the 128-bit mask (m0: j < 64) is set.
__device__ inline void flip_signs(float (&v)[128], uint64_t m0, uint64_t m1) {
#pragma unroll
  for (int j = 0; j < 128; ++j) {
    const uint64_t m = j < 64 ? m0 : m1;
    const uint32_t bit = (uint32_t)(m >> (j & 63)) & 1u;
    v[j] = __uint_as_float(__float_as_uint(v[j]) ^ (bit << 31));
  }
}

// Loads row (b, h, t) of x as fp32 (zeros for a lane past the last token).
__device__ inline void load_row(const EncodeArgs& a, int b, int h, int t, bool valid,
                                float (&v)[128]) {
  const int64_t off = (int64_t)b * a.s0 + (int64_t)h * a.s1 + (int64_t)(valid ? t : 0) * a.s2;
  if (a.is_bf16) {
    const uint16_t* row = static_cast<const uint16_t*>(a.x) + off;
    if (a.vec16) {
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const uint4 w = reinterpret_cast<const uint4*>(row)[k];
        const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          v[8 * k + 2 * m] = __uint_as_float(ws[m] << 16);
          v[8 * k + 2 * m + 1] = __uint_as_float(ws[m] & 0xffff0000u);
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < 128; ++j) v[j] = bf16_to_f32(row[j]);
    }
  } else {
    const float* row = static_cast<const float*>(a.x) + off;
    if (a.vec16) {
#pragma unroll
      for (int k = 0; k < 32; ++k) {
        const float4 w = reinterpret_cast<const float4*>(row)[k];
        v[4 * k] = w.x;
        v[4 * k + 1] = w.y;
        v[4 * k + 2] = w.z;
        v[4 * k + 3] = w.w;
      }
    } else {
#pragma unroll
      for (int j = 0; j < 128; ++j) v[j] = row[j];
    }
  }
  if (!valid) {
#pragma unroll
    for (int j = 0; j < 128; ++j) v[j] = 0.0f;
  }
}

// ---------------------------------------------------------------- encoder
// Four lanes per token.  A wavefront takes 16 tokens at a time (column col =
// L % 16 of the matrix products) and lane group g = L / 16 of a token holds
// its coordinates 32 g .. 32 g + 31.
//
// Rotation: with k = 8 k_hi + k_lo (Sylvester order) H_128 = H_16 (x) H_8,
// so R x = H diag(s) x is, for each k_lo, the 16 x 16 product
//   V_klo[r_hi][token] = sum_khi H_16[r_hi][k_hi] s_(8 k_hi + k_lo) x_(8 k_hi + k_lo)
// -- one v_mfma_f32_16x16x16_bf16 whose operands are exact (+-1 and the bf16
// input; an fp32 input is split into three bf16 terms, each product exact in
// the fp32 accumulation) -- followed by the 8-point transform over k_lo in
// registers: y_(8 r_hi + r_lo) = sum_klo H_8[r_lo][k_lo] V_klo[r_hi].  The
// product's lane layout leaves rows r_hi = 4 g .. 4 g + 3 in lane group g,
// that is, coordinates 32 g .. 32 g + 31 again.
//
// Triplets: through the wavefront's rows of LDS, lane group g takes the
// coordinates of triplets 10 g .. 10 g + 9 and of triplet 40 + g (g < 3), so
// that the triplet code runs with compile-time register indices; each field
// is OR-ed into the token's record in LDS at its bit offset, and the
// records are stored word by word, 16 tokens (64 bytes) a store.
constexpr int kTokTile = 16;                 // tokens of a wavefront tile
constexpr int kEncWaves = 4;
constexpr int kEncThreads = 64 * kEncWaves;  // 64 tokens per workgroup
constexpr int kXRow = kHeadDim + 4;          // floats per token row of the exchange rows

typedef short short4v __attribute__((ext_vector_type(4)));
typedef float floatx4e __attribute__((ext_vector_type(4)));

// bf16 bits of v rounded to nearest even (finite inputs)
__device__ inline uint32_t bf16_rne(float v) {
  const uint32_t u = __float_as_uint(v);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// H_8 (Sylvester order, unnormalized) on eight registers.
__device__ inline void wht8(float (&v)[8]) {
#pragma unroll
  for (int h = 1; h < 8; h <<= 1)
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (!(i & h)) {
        const float p = v[i], q = v[i + h];
        v[i] = p + q;
        v[i + h] = p - q;
      }
}

// y = H diag(s) x for the lane's token, coordinates 32 g + m in y[m]; the
// input is given as bf16 terms: bterm(t, k_lo) returns the B operand
// {x_(32 g + 8 e + k_lo) : e = 0..3} of term t.  amat[k_lo] holds the A
// operands {H_16[L % 16][4 g + e] s_(32 g + 8 e + k_lo)}.
template <int NT, class BTerm>
__device__ inline void rotate16(const short4v (&amat)[8], BTerm&& bterm, float (&y)[32]) {
  floatx4e d[8];
#pragma unroll
  for (int kl = 0; kl < 8; ++kl) {
    d[kl] = floatx4e{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int t = 0; t < NT; ++t)
      d[kl] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(amat[kl], bterm(t, kl), d[kl], 0, 0, 0);
  }
  // rows r_hi = 4 g + r: the 8-point transform over k_lo
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    float v[8];
#pragma unroll
    for (int kl = 0; kl < 8; ++kl) v[kl] = d[kl][r];
    wht8(v);
#pragma unroll
    for (int rl = 0; rl < 8; ++rl) y[8 * r + rl] = v[rl];
  }
}

// The three bf16 terms of an fp32 value: hi = bf16(x), mid = bf16(x - hi),
// lo = bf16(x - hi - mid), whose sum is x to about 2^-24 relative.
__device__ inline void split3(float x, uint32_t& hi, uint32_t& mid, uint32_t& lo) {
  hi = bf16_rne(x);
  const float r1 = x - __uint_as_float(hi << 16);
  mid = bf16_rne(r1);
  const float r2 = r1 - __uint_as_float(mid << 16);
  lo = bf16_rne(r2);
}

// Sum of a value over the four lane groups of a token (lanes L, L ^ 16,
// L ^ 32, L ^ 48), the same in all four.
__device__ inline float groups_sum(float x) {
  x += __shfl_xor(x, 16, 64);
  x += __shfl_xor(x, 32, 64);
  return x;
}

// Three workgroups a CU for bf16 input at b_dir = 5 (LDS 52 KB each, at
// most 168 registers a lane); smaller tables leave room for four by LDS.
// MT: each wavefront takes a.tiles tiles, so that a large direction table
// serves many tokens.
template <int BD, int BN, bool F32, bool MT>
__global__ __launch_bounds__(kEncThreads, BD == 5 && !F32 ? 3 : 2) void encode_part_kernel(EncodeArgs a) {
  constexpr int K = 1 << BD, R = 1 << BN;
  constexpr int FWD = 2 * BD;                         // xi | eta << BD
  constexpr int BT = FWD + BN;                        // + rho << 2 BD: one field per triplet
  constexpr int WI = (kNTri * BT + 31) / 32;
  static_assert(WI <= kXRow, "a record fits the first words of a token's row");

  constexpr int KP = K + 2;                           // padded side of the direction table
  // Direction table, padded by one cell on every side: entry (i, j), i, j in
  // [-1, K], at (i + 1) + KP (j + 1) holds n(c_xi[i'], c_xi[j']) and the code
  // pair i' | j' << BD of the clamped cell (i', j'), so the 3x3 neighbourhood
  // of a seed is nine reads at constant offsets, and a clamped neighbour is
  // the same candidate as the cell it clamps to.
  __shared__ floatx4 lut[KP * KP];
  __shared__ float cxi[K], midp[K + 1], crho[R], mid_rho[R];
  __shared__ int guess_bad;
  // per wavefront: the exchange rows of its 16 tokens; once a tile's
  // coordinates are in registers, the first words of a token's row hold its
  // record (a separate array would keep the workgroup above a third of the
  // CU's LDS)
  __shared__ __attribute__((aligned(16))) float xrows[kEncWaves][kTokTile][kXRow];

  const int tid = threadIdx.x, L = tid & 63, wave = tid >> 6;
  const int col = L & 15, g = L >> 4;
  const int h = blockIdx.y, b = blockIdx.z;
  const size_t plane = (size_t)b * a.H + h;
  // the workgroup's 64 n_tiles tokens: tile it of wavefront w is tokens
  // base + 16 (4 it + w) + (0..15)
  const int n_tiles = MT ? a.tiles : 1;
  const int base = blockIdx.x * (kEncWaves * kTokTile * n_tiles);
  auto token_of = [&](int it) { return base + kTokTile * (kEncWaves * it + wave) + col; };

  // ---- A operands of H diag(s) (and of H diag(s')):
  // {H_16[col][4 g + e] s_(32 g + 8 e + k_lo)} as bf16 +-1, from the lane
  // group's 32 sign bits
  auto a_operands = [&](const uint32_t (&mask)[4], short4v (&am)[8]) __attribute__((always_inline)) {
    // bit 8 e + k_lo of x: the sign of entry e of the k_lo operand
    uint32_t x = g == 0 ? mask[0] : g == 1 ? mask[1] : g == 2 ? mask[2] : mask[3];
#pragma unroll
    for (int e = 0; e < 4; ++e) x ^= (uint32_t)(__builtin_popcount(col & (4 * g + e)) & 1) * (0xffu << (8 * e));
#pragma unroll
    for (int kl = 0; kl < 8; ++kl) {
      const uint32_t y = x >> kl;
      const uint32_t w0 = 0x3f803f80u | ((y << 15) & 0x8000u) | ((y << 23) & 0x80000000u);
      const uint32_t w1 = 0x3f803f80u | ((y >> 1) & 0x8000u) | ((y << 7) & 0x80000000u);
      am[kl] = __builtin_bit_cast(short4v, make_uint2(w0, w1));
    }
  };
  short4v am[8];
  a_operands(a.smask, am);

  // ---- the lane's 32 coordinates of tile it (bf16 input: words xw, pairs
  // (2 j, 2 j + 1); fp32 input: xf), zeros past the last token
  uint32_t xw[F32 ? 1 : 16];
  float xf[F32 ? 32 : 1];
  auto load_x = [&](int it) __attribute__((always_inline)) {
    const int t = token_of(it);
    const bool valid = t < a.T;
    const int64_t off = (int64_t)b * a.s0 + (int64_t)h * a.s1 + (int64_t)(valid ? t : 0) * a.s2 + 32 * g;
    if constexpr (!F32) {
      const uint16_t* row = static_cast<const uint16_t*>(a.x) + off;
      if (a.vec16) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const uint4 w = reinterpret_cast<const uint4*>(row)[k];
          xw[4 * k] = valid ? w.x : 0u;
          xw[4 * k + 1] = valid ? w.y : 0u;
          xw[4 * k + 2] = valid ? w.z : 0u;
          xw[4 * k + 3] = valid ? w.w : 0u;
        }
      } else {
#pragma unroll
        for (int j = 0; j < 16; ++j)
          xw[j] = valid ? (uint32_t)row[2 * j] | ((uint32_t)row[2 * j + 1] << 16) : 0u;
      }
    } else {
      const float* row = static_cast<const float*>(a.x) + off;
      if (a.vec16) {
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const float4 w = reinterpret_cast<const float4*>(row)[k];
          xf[4 * k] = valid ? w.x : 0.0f;
          xf[4 * k + 1] = valid ? w.y : 0.0f;
          xf[4 * k + 2] = valid ? w.z : 0.0f;
          xf[4 * k + 3] = valid ? w.w : 0.0f;
        }
      } else {
#pragma unroll
        for (int j = 0; j < 32; ++j) xf[j] = valid ? row[j] : 0.0f;
      }
    }
  };
  load_x(0);                           // issued before the tables are built

  // ---- tables: codebooks, cell boundaries, decoded directions
  if (tid < K) cxi[tid] = a.cb.xi[tid];
  if (tid < R) crho[tid] = a.cb.rho[tid];
  if (tid == 0) {
    guess_bad = 0;
    midp[0] = -INFINITY;
    midp[K] = INFINITY;
  }
  __syncthreads();
  if (tid < K - 1) {
    const float m = 0.5f * (cxi[tid] + cxi[tid + 1]);
    midp[tid + 1] = m;
    // uniform grid boundaries b_k = -1 + 2 (k + 1) / K; the one-step
    // correction is exact when b_(k-1) <= mid_k < b_(k+1) (with a margin
    // for the rounding of the grid index)
    const float lo = tid > 0 ? -1.0f + 2.0f * tid / K : -INFINITY;
    const float hi = tid + 2 < K ? -1.0f + 2.0f * (tid + 2) / K : INFINITY;
    if (!(m >= lo + 1e-5f && m < hi - 1e-5f)) guess_bad = 1;
  }
  if (tid < R - 1) mid_rho[tid] = 0.5f * (crho[tid] + crho[tid + 1]);
  for (int e = tid; e < KP * KP; e += kEncThreads) {
    // Eq. 6 with the fold of App. C.7, then normalization onto S^2.
    const int ci = min(max(e % KP - 1, 0), K - 1), cj = min(max(e / KP - 1, 0), K - 1);
    const float xi = cxi[ci], eta = cxi[cj];
    const float z = 1.0f - fabsf(xi) - fabsf(eta);
    float x = xi, y = eta;
    if (z < 0.0f) {
      x = (xi >= 0.0f ? 1.0f : -1.0f) * (1.0f - fabsf(eta));
      y = (eta >= 0.0f ? 1.0f : -1.0f) * (1.0f - fabsf(xi));
    }
    const float n = fmaxf(sqrtf(x * x + y * y + z * z), kEps);
    lut[e] = floatx4{x / n, y / n, z / n, __uint_as_float((uint32_t)(ci | (cj << BD)))};
  }
  __syncthreads();
  // uniform: a scalar branch, not a masked one
  const bool guess_ok = __builtin_amdgcn_readfirstlane(guess_bad) == 0;
  float mr[R > 1 ? R - 1 : 1];
#pragma unroll
  for (int k = 0; k < R - 1; ++k) mr[k] = mid_rho[k];

  float* xr = xrows[wave][col];
  uint32_t* rec = reinterpret_cast<uint32_t*>(xr);
  const bool scalar = a.rounding == OCTO_ROUND_SCALAR;     // kernel argument: uniform
  const bool has_tail = g < 3;
  // coordinate j of the lane's 32
  auto xval = [&](int j) __attribute__((always_inline)) {
    if constexpr (F32) return xf[j];
    else return __uint_as_float(j & 1 ? xw[j >> 1] & 0xffff0000u : xw[j >> 1] << 16);
  };
#pragma unroll 1
  for (int it = 0; it < n_tiles; ++it) {
  const int t = token_of(it);
  const bool valid = t < a.T;
  // ---- gamma, rotation, scaling (Sec. 3.1)
  float ss[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int j = 0; j < 32; ++j) ss[j & 3] = fmaf(xval(j), xval(j), ss[j & 3]);
  const float gamma = sqrtf(groups_sum((ss[0] + ss[1]) + (ss[2] + ss[3])));
  float y[32];
  if constexpr (!F32) {
    rotate16<1>(am, [&](int, int kl) {
      // {x_(8 e + kl)}: halves kl % 2 of words 4 e + kl / 2
      const uint32_t sel = kl & 1 ? 0x07060302u : 0x05040100u;
      const uint32_t p01 = __builtin_amdgcn_perm(xw[4 + (kl >> 1)], xw[kl >> 1], sel);
      const uint32_t p23 = __builtin_amdgcn_perm(xw[12 + (kl >> 1)], xw[8 + (kl >> 1)], sel);
      return __builtin_bit_cast(short4v, make_uint2(p01, p23));
    }, y);
  } else {
    uint32_t tw[3][16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      uint32_t h0, m0, l0, h1, m1, l1;
      split3(xf[2 * j], h0, m0, l0);
      split3(xf[2 * j + 1], h1, m1, l1);
      tw[0][j] = h0 | (h1 << 16);
      tw[1][j] = m0 | (m1 << 16);
      tw[2][j] = l0 | (l1 << 16);
    }
    rotate16<3>(am, [&](int tt, int kl) {
      const uint32_t sel = kl & 1 ? 0x07060302u : 0x05040100u;
      const uint32_t p01 = __builtin_amdgcn_perm(tw[tt][4 + (kl >> 1)], tw[tt][kl >> 1], sel);
      const uint32_t p23 = __builtin_amdgcn_perm(tw[tt][12 + (kl >> 1)], tw[tt][8 + (kl >> 1)], sel);
      return __builtin_bit_cast(short4v, make_uint2(p01, p23));
    }, y);
  }
  const float scale = kInvSqrtD / fmaxf(gamma, kEps);
  if (it + 1 < n_tiles) load_x(it + 1);  // the next tile's coordinates

  // ---- to the triplet layout: coordinates 30 g .. 30 g + 29 (triplets
  // 10 g .. 10 g + 9) and 120 + 3 g .. 122 + 3 g (triplet 40 + g; the zero
  // pad at 128)
#pragma unroll
  for (int j = 0; j < 32; j += 4)
    *reinterpret_cast<floatx4*>(&xr[32 * g + j]) =
        floatx4{y[j] * scale, y[j + 1] * scale, y[j + 2] * scale, y[j + 3] * scale};
  if (g == 0) *reinterpret_cast<floatx4*>(&xr[kHeadDim]) = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  float v[33];
#pragma unroll
  for (int j = 0; j < 30; j += 2) {
    const float2 p = *reinterpret_cast<const float2*>(&xr[30 * g + j]);
    v[j] = p.x;
    v[j + 1] = p.y;
  }
#pragma unroll
  for (int j = 0; j < 3; ++j) v[30 + j] = has_tail ? xr[120 + 3 * g + j] : 0.0f;
  // the row's coordinates are read: its first WI words become the empty
  // record (lane group g clears words g, g + 4, ..)
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
  for (int w0 = 0; w0 < WI; w0 += 4)
    if (w0 + g < WI) rec[w0 + g] = 0u;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  // ---- triplets: octahedral map, seeds, joint rounding, fields
  StaticFor<0, 11>::run([&](auto mc) {
    constexpr int m = decltype(mc)::value;
    // one triplet at a time: keeps the scheduler from interleaving the
    // iterations (and their table reads) into a register spill
    __builtin_amdgcn_sched_barrier(0);
    if (m == 10 && !has_tail) return;
    const int i = m < 10 ? 10 * g + m : 40 + g;          // the triplet
    const float tx = v[3 * m], ty = v[3 * m + 1], tz = v[3 * m + 2];
    // Eq. 5 on the L1-normalized direction, sign(0) = +1.
    const float inv_l1 = __builtin_amdgcn_rcpf(fmaxf(fabsf(tx) + fabsf(ty) + fabsf(tz), kEps));
    const float px = tx * inv_l1, py = ty * inv_l1, pz = tz * inv_l1;
    float xi = px, eta = py;
    if (pz < 0.0f) {
      xi = (px >= 0.0f ? 1.0f : -1.0f) * (1.0f - fabsf(py));
      eta = (py >= 0.0f ? 1.0f : -1.0f) * (1.0f - fabsf(px));
    }
    int sx, sy;
    if (guess_ok) {
      sx = seed_guess<K>(midp, xi);
      sy = seed_guess<K>(midp, eta);
    } else {
      sx = seed_search<K>(midp, xi);
      sy = seed_search<K>(midp, eta);
    }
    // corner (-1, -1) of the seed's neighbourhood; candidate (dx, dy) sits at
    // offset (dx + 1) + KP (dy + 1)
    const floatx4* nbh = &lut[sx + KP * sy];
    floatx4 n0 = nbh[1 + KP];
    pin(n0);
    uint32_t code = __float_as_uint(n0.w);
    int ir;
    if (scalar) {
      ir = rho_index<R>(mr, sqrtf(tx * tx + ty * ty + tz * tz));
    } else {
      // Seed first, then the other eight neighbours row-major (dx outer);
      // only a strictly larger s replaces the incumbent.
      float best = tx * n0.x + ty * n0.y + tz * n0.z;
#pragma unroll
      for (int dx = 0; dx < 3; ++dx)
#pragma unroll
        for (int dy = 0; dy < 3; ++dy) {
          if (dx == 1 && dy == 1) continue;
          floatx4 n = nbh[dx + KP * dy];
          pin(n);
          const float s = tx * n.x + ty * n.y + tz * n.z;
          const bool up = s > best;
          best = up ? s : best;
          code = up ? __float_as_uint(n.w) : code;
        }
      ir = rho_index<R>(mr, best);
    }
    // the field at bit i B_tri of the record (LSB-first stream)
    {
      const uint32_t f = code | ((uint32_t)ir << FWD);
      const int pos = i * BT, w = pos >> 5, sh = pos & 31;
      __hip_atomic_fetch_or(&rec[w], f << sh, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      if (sh + BT > 32)
        __hip_atomic_fetch_or(&rec[w + 1], f >> (32 - sh), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
    if (a.qjl) {
      // rotated-frame residual r = u - u^ (Sec. 3.6), over the real coordinates
      floatx4 nb = n0;
      if (!scalar) {
        nb = lut[(code & (K - 1)) + 1 + KP * ((code >> BD) + 1)];
        pin(nb);
      }
      const float rho = crho[ir];
      v[3 * m] = tx - rho * nb.x;
      v[3 * m + 1] = ty - rho * nb.y;
      v[3 * m + 2] = tz - rho * nb.z;
    }
  });
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  // ---- stores: word w of 64 consecutive tokens is 256 contiguous bytes;
  // lane group g stores words g, g + 4, .. of the 16 tokens
  const int tc = a.token_offset + t;
  if (valid) {
#pragma unroll
    for (int w0 = 0; w0 < WI; w0 += 4)
      if (w0 + g < WI) a.idx[tile_word(plane, a.capacity, tc, w0 + g, WI)] = rec[w0 + g];
    if (g == 0) a.gamma[plane * a.capacity + tc] = gamma;
  }

  // ---- QJL: sigma = sign(H diag(s') r), gamma_r = fp16(||r||)
  if (a.qjl) {
    // the records are read (stored) before the rows take the residual
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // the residual back to coordinate order (the pad is not written)
#pragma unroll
    for (int j = 0; j < 30; j += 2) *reinterpret_cast<float2*>(&xr[30 * g + j]) = make_float2(v[j], v[j + 1]);
    if (has_tail) {
#pragma unroll
      for (int j = 0; j < 3; ++j)
        if (120 + 3 * g + j < kHeadDim) xr[120 + 3 * g + j] = v[30 + j];
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    float rv[32];
#pragma unroll
    for (int j = 0; j < 32; j += 4) {
      const floatx4 q = *reinterpret_cast<const floatx4*>(&xr[32 * g + j]);
      rv[j] = q[0];
      rv[j + 1] = q[1];
      rv[j + 2] = q[2];
      rv[j + 3] = q[3];
    }
    float rs[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int j = 0; j < 32; ++j) rs[j & 3] = fmaf(rv[j], rv[j], rs[j & 3]);
    const float rn = sqrtf(groups_sum((rs[0] + rs[1]) + (rs[2] + rs[3])));
    uint32_t tw[3][16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      uint32_t h0, m0, l0, h1, m1, l1;
      split3(rv[2 * j], h0, m0, l0);
      split3(rv[2 * j + 1], h1, m1, l1);
      tw[0][j] = h0 | (h1 << 16);
      tw[1][j] = m0 | (m1 << 16);
      tw[2][j] = l0 | (l1 << 16);
    }
    short4v aq[8];
    a_operands(a.qmask, aq);
    float z[32];
    rotate16<3>(aq, [&](int tt, int kl) {
      const uint32_t sel = kl & 1 ? 0x07060302u : 0x05040100u;
      const uint32_t p01 = __builtin_amdgcn_perm(tw[tt][4 + (kl >> 1)], tw[tt][kl >> 1], sel);
      const uint32_t p23 = __builtin_amdgcn_perm(tw[tt][12 + (kl >> 1)], tw[tt][8 + (kl >> 1)], sel);
      return __builtin_bit_cast(short4v, make_uint2(p01, p23));
    }, z);
    uint32_t sw = 0u;
#pragma unroll
    for (int j = 0; j < 32; ++j) sw |= (uint32_t)(z[j] < 0.0f) << j;
    if (valid) {
      a.qjl_bits[tile_word(plane, a.capacity, tc, g, 4)] = sw;
      if (g == 0) {
        const _Float16 hr = (_Float16)rn;
        a.gamma_r[plane * a.capacity + tc] = __builtin_bit_cast(uint16_t, hr);
      }
    }
  }
  if (MT) {
    // the rows and records are read before the next tile writes them
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
  }
}

// The group-wise value codec (group = 16 or 32): one lane per token, u = R x
// in registers as above, then per group of GS coordinates the range, the
// E4M3 step size, the BF16 zero-point and the codes (the quantizer of
// "Quantized Keys Steal Attention", Sec. 3 and Sec. 4.3, as the value codec
// of the OCTOPUS experiments, Sec. 4).  Every decision is an fp32 operation:
// the division is the correctly rounded one, rint rounds half to even.
template <int VB, int GS>
__global__ __launch_bounds__(kThreads, 2) void group_encode_kernel(EncodeArgs a) {
  constexpr int G = kHeadDim / GS, WC = VB * kHeadDim / 32, W = group_record_words(VB, GS);
  constexpr float kLevels = (float)((1 << VB) - 1);
  const int tid = threadIdx.x;
  const int h = blockIdx.y, b = blockIdx.z;
  const int t = blockIdx.x * kThreads + tid;
  const bool valid = t < a.T;
  const size_t plane = (size_t)b * a.H + h;
  const int ln = tid & 63;
  const uint64_t sm0 = __ballot(splitmix_sign(a.seed, ln) < 0.0f);
  const uint64_t sm1 = __ballot(splitmix_sign(a.seed, ln + 64) < 0.0f);
  float v[128];
  load_row(a, b, h, t, valid, v);
  flip_signs(v, sm0, sm1);
  wht128_regs(v);
#pragma unroll
  for (int j = 0; j < 128; ++j) v[j] *= kInvSqrtD;

  uint32_t rec[W];
#pragma unroll
  for (int w = 0; w < W; ++w) rec[w] = 0u;
#pragma unroll
  for (int gi = 0; gi < G; ++gi) {
    __builtin_amdgcn_sched_barrier(0);   // one group at a time (no interleaving spills)
    float mn = v[gi * GS], mx = mn;
#pragma unroll
    for (int j = 1; j < GS; ++j) {
      mn = fminf(mn, v[gi * GS + j]);
      mx = fmaxf(mx, v[gi * GS + j]);
    }
    mn += 0.0f;                          // a zero minimum is stored as +0
    const uint32_t s8 = e4m3_rne((mx - mn) / kLevels);
    const float dh = e4m3_value(s8);
    const uint32_t z16 = bf16_rne(mn);
    const float zh = __uint_as_float(z16 << 16);
#pragma unroll
    for (int j = 0; j < GS; ++j) {
      const int c = gi * GS + j;
      const float qf = fminf(fmaxf(rintf((v[c] - zh) / dh), 0.0f), kLevels);
      const uint32_t q = dh > 0.0f ? (uint32_t)qf : 0u;
      const int pos = c * VB, w = pos >> 5, sh = pos & 31;
      rec[w] |= q << sh;
      if (sh + VB > 32) rec[w + 1] |= q >> (32 - sh);
    }
    rec[WC + gi / 4] |= s8 << (8 * (gi % 4));
    rec[WC + G / 4 + gi / 2] |= z16 << (16 * (gi % 2));
  }
  if (valid) {
    const int tc = a.token_offset + t;
#pragma unroll
    for (int w = 0; w < W; ++w) a.idx[tile_word(plane, a.capacity, tc, w, W)] = rec[w];
  }
}

constexpr int kCUs = 256;                     // compute units of the MI355X

template <int BD, int BN>
void launch(const EncodeArgs& a, hipStream_t st) {
  // b_dir >= 5: the direction table is large and costs a workgroup as much
  // as several tiles, so each wavefront takes as many tiles as fill the
  // chip with one round of resident workgroups (three a CU with bf16 input
  // at b_dir = 5, two with fp32 input, one at b_dir = 6, bound by the LDS
  // and the registers)
  constexpr bool kMT = BD >= 5;
  EncodeArgs args = a;
  args.tiles = 1;
  if (kMT) {
    const int per_cu = BD >= 6 ? 1 : (a.is_bf16 ? 3 : 2);
    const int64_t tok = (int64_t)a.T * a.H * a.B;
    const int64_t slots = (int64_t)kCUs * per_cu * kEncWaves * kTokTile;
    args.tiles = (int)std::max<int64_t>(1, (tok + slots - 1) / slots);
  }
  const void* fn = a.is_bf16 ? reinterpret_cast<const void*>(&encode_part_kernel<BD, BN, false, kMT>)
                             : reinterpret_cast<const void*>(&encode_part_kernel<BD, BN, true, kMT>);
  const int tok_wg = kEncWaves * kTokTile * args.tiles;
  void* kargs[] = {&args};
  (void)hipLaunchKernel(fn, dim3((a.T + tok_wg - 1) / tok_wg, a.H, a.B), dim3(kEncThreads), kargs, 0, st);
}

template <int VB, int GS>
void launch_group(const EncodeArgs& a, hipStream_t st) {
  dim3 grid((a.T + kThreads - 1) / kThreads, a.H, a.B);
  hipLaunchKernelGGL((group_encode_kernel<VB, GS>), grid, dim3(kThreads), 0, st, a);
}

}  // namespace
}  // namespace octo

extern "C" octo_status octo_encode(const octo_codec_desc* codec, const void* x, int32_t x_dtype,
                                   int32_t B, int32_t H, int32_t T, const int64_t x_strides[4],
                                   const octo_cache_view* dst, int32_t token_offset,
                                   hipStream_t stream) {
  using namespace octo;
  clear_error();
  Codec c;
  octo_status s = resolve_codec(codec, "octo_encode", &c, true, true);
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
  a.vec16 = ((uintptr_t)x % 16 == 0) && ((x_strides[0] * esz) % 16 == 0) &&
            ((x_strides[1] * esz) % 16 == 0) && ((x_strides[2] * esz) % 16 == 0);
  a.B = B;
  a.H = H;
  a.T = T;
  a.cb = c.wcb;
  a.seed = c.seed;
  a.qjl = c.qjl;
  a.rounding = c.rounding;
  a.idx = dst->idx;
  a.gamma = dst->gamma;
  a.qjl_bits = dst->qjl;
  a.gamma_r = dst->gamma_r;
  a.capacity = dst->capacity;
  a.token_offset = token_offset;
  for (int w = 0; w < 4; ++w) {
    a.smask[w] = a.qmask[w] = 0u;
    for (int j = 0; j < 32; ++j) {
      a.smask[w] |= (uint32_t)(splitmix_sign(c.seed, 32 * w + j) < 0.0f) << j;
      a.qmask[w] |= (uint32_t)(splitmix_sign(c.seed, kHeadDim + 32 * w + j) < 0.0f) << j;
    }
  }

  if (c.group) {
    switch (c.bits * 100 + c.group) {
      case 216: launch_group<2, 16>(a, stream); break;
      case 232: launch_group<2, 32>(a, stream); break;
      case 316: launch_group<3, 16>(a, stream); break;
      case 332: launch_group<3, 32>(a, stream); break;
      case 416: launch_group<4, 16>(a, stream); break;
      case 432: launch_group<4, 32>(a, stream); break;
      default: return fail(OCTO_ERR_UNSUPPORTED, "octo_encode: group codec not compiled");
    }
    return check_launch("octo_encode");
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
    default: return fail(OCTO_ERR_UNSUPPORTED, "octo_encode: split not compiled");
  }
  return check_launch("octo_encode");
}
