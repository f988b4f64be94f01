// Internal declarations shared by the OCTOPUS HIP library sources.
//
// The method is the one of "OCTOPUS: Optimized KV Cache for Transformers via
// Octahedral Parametrization Under optimal Squared error quantization"
// (arXiv 2605.21226), Sec. 3.  This header holds the resolved codec
// parameters, the host-side status plumbing and the small device helpers
// (sign generator, wavefront Walsh-Hadamard transform, bit-field access) that
// the encode, decode and chunk kernels share.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "octopus.h"

namespace octo {

constexpr int kHeadDim = 128;            // d supported by the kernels
constexpr int kNTri = 43;                // ceil(128 / 3) triplets (Sec. 3.2)
constexpr int kPadDim = 3 * kNTri;       // 129: u zero-padded to whole triplets
constexpr float kEps = 1e-20f;           // the eps-safe divisor of Sec. 3.1 / 3.2
constexpr int kWave = 64;


constexpr int kMaxXi = 32;            // 2^b_dir centroids, b_dir <= 5
constexpr int kMaxRho = 16;           // 2^b_nrm centroids, b_nrm <= 4

// The codebook values, passed to the kernels by value (kernel arguments
// arrive with the launch: no dependent load of a table before the kernels
// can build their LDS tables).  Unused entries are zero.
struct Codebook {
  float xi[kMaxXi];
  float rho[kMaxRho];
};
// The same for the encoder and the explicit reconstruction, which also take
// the splits of the (b + delta, b - delta) sweep (Sec. 3.3), up to 2^6
// centroids on either side.
constexpr int kMaxWide = 64;
struct WideCodebook {
  float xi[kMaxWide];
  float rho[kMaxWide];
};

// A codec with its bit split resolved (Sec. 3.3: B_tri = 2 b_dir + b_nrm),
// or the group-wise value codec (group = 16 or 32; b_dir = b_nrm = 0).
struct Codec {
  int group;            // 0: OCTOPUS; else the group size g of the value codec
  int bits;             // b of the group codec (the OCTOPUS codec: the mean
                        // (b_dir + b_nrm) / 2, b of a (b + delta, b - delta) split)
  int b_dir, b_nrm;     // bits per octahedral coordinate / per triplet norm
  int K;                // 2^b_dir entries of C_xi
  int R;                // 2^b_nrm entries of C_rho
  int w_idx, w_qjl;     // 32-bit words per token of each stream
  int qjl;
  int rounding;
  uint64_t seed;
  Codebook cb;          // the C_xi, C_rho values read from the descriptor
                        // (splits the attention kernels take)
  WideCodebook wcb;     // the same, for any split the encoder takes
};

// ---------------------------------------------------------------- host side
// Thread-local message behind octo_last_error(); returns `s` for chaining.
octo_status fail(octo_status s, const char* fmt, ...);
void clear_error();
// Validates a descriptor and resolves its split; nothing on the device is read.
// need_tables: the codebook pointers must be set and are read (every compute
// entry point): finite, ascending values.
// any_split: also the splits of the (b + delta, b - delta) sweep that only the
// encoder and the explicit reconstruction are compiled for.
octo_status resolve_codec(const octo_codec_desc* desc, const char* what, Codec* out,
                          bool need_tables = true, bool any_split = false);
// Validates a cache view against a codec (pointers, sizes, alignment).
octo_status check_cache(const octo_cache_view* v, const Codec& c, const char* what);
// Maps the last HIP launch error to OCTO_ERR_HIP.
octo_status check_launch(const char* what);

inline int words_for_bits(int bits) { return (bits + 31) / 32; }

// Words of one group-codec record: 128 b-bit codes, 128/g E4M3 scales and
// 128/g BF16 zero-points.
constexpr int group_record_words(int bits, int g) { return (kHeadDim * bits + 24 * (kHeadDim / g)) / 32; }

// ---------------------------------------------------------------- device side
// SplitMix64 output j of the generator started at `seed` (Steele, Lea and
// Flood, OOPSLA 2014): the sign s_j of the rotation R = H diag(s) is -1 when
// bit 63 is set.  j < d gives s, d <= j < 2d gives the QJL signs s'.
__host__ __device__ inline float splitmix_sign(uint64_t seed, uint32_t j) {
  uint64_t z = seed + (uint64_t)(j + 1) * 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  z = z ^ (z >> 31);
  return (z >> 63) ? -1.0f : 1.0f;
}

// The value of lane L ^ m (m a power of two below 64, known after
// unrolling): a DPP quad permutation for m = 1 and 2, a cross-lane read
// otherwise.
__device__ __forceinline__ float lane_xor(float v, int m) {
  if (m == 1) return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, true));
  if (m == 2) return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, true));
  return __shfl_xor(v, m, 64);
}

// One cross-lane butterfly of a Walsh-Hadamard stage: v + p in the lane of
// the pair with the stage's bit clear, p - v in its partner (p the other
// lane's value), as one fused multiply-add by the lane's sign sg (+1 or
// -1).  The product by +-1 is exact and the sum is rounded once, so the
// result is the add or subtract itself.
__device__ __forceinline__ float xbfly(float v, float p, float sg) { return fmaf(sg, v, p); }

// Unnormalized Walsh-Hadamard transform of a 128-vector held by one
// wavefront, lane l owning coordinates l (a) and l + 64 (b).  Natural
// (Sylvester) order: H[i][j] = (-1)^popcount(i & j).  The stride-64 butterfly
// is lane-local, strides 32..1 exchange across lanes.
__device__ inline void wht128(float& a, float& b) {
  const int lane = threadIdx.x & 63;
  float s = a + b, t = a - b;
  a = s;
  b = t;
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    const float pa = lane_xor(a, m), pb = lane_xor(b, m);
    const float sg = (lane & m) ? -1.0f : 1.0f;
    a = xbfly(a, pa, sg);
    b = xbfly(b, pb, sg);
  }
}

// Reductions over the four 16-lane rows of a wavefront (lanes L, L ^ 16,
// L ^ 32, L ^ 48) with the lane-half and row swaps, no LDS round trip.  Both
// halves of each swap are combined in the same order in every lane, so all
// four lanes hold the same bits.
__device__ inline float rows_max(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ inline float rows_sum(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

__device__ inline float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, 64));
  return v;
}

// bf16 -> fp32 is exact: the bf16 bits are the high half of the fp32 bits.
__device__ inline float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// E4M3 (4 exponent bits, bias 7, 3 mantissa bits, no infinities, largest
// finite value 448) code of a non-negative finite fp32 value: round to
// nearest, ties to the even code, saturating at 448.  Codes 0..8 are the
// multiples of 2^-9 up to 2^-6 (the subnormals and the smallest normal);
// above, the fp32 exponent and top mantissa bits are the code once the
// bias is moved from 127 to 7.
__device__ inline uint32_t e4m3_rne(float x) {
  if (!(x < 448.0f)) return 0x7Eu;
  if (x < 0.015625f) return (uint32_t)rintf(x * 512.0f);
  const uint32_t u = __float_as_uint(x);
  return ((u + 0x7FFFFu + ((u >> 20) & 1u)) >> 20) - (120u << 3);
}
// Exact fp32 value of an E4M3 code 0..0x7E.
__device__ inline float e4m3_value(uint32_t c) {
  return c >= 8u ? __uint_as_float((c + (120u << 3)) << 20) : (float)c * 0.001953125f;
}
// BF16 bit pattern of a finite fp32 value, round to nearest even.
__device__ inline uint32_t bf16_rne(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Workgroup barrier that orders LDS only: it waits for this wave's LDS
// operations but leaves its global loads in flight (a full __syncthreads
// also waits for every outstanding global load).
__device__ inline void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Field of WIDTH bits at bit offset POS of a little-endian LSB-first stream
// held in registers (POS and WIDTH become constants after unrolling).
template <int WIDTH>
__device__ inline uint32_t field(const uint32_t* w, int pos) {
  const int wi = pos >> 5, sh = pos & 31;
  const uint32_t v = sh + WIDTH > 32 ? __builtin_amdgcn_alignbit(w[wi + 1], w[wi], sh) : w[wi] >> sh;
  return v & ((1u << WIDTH) - 1u);
}

// Word index of word `w` of token `t` in plane `plane` of a tile-64 stream
// with W words per token: each 64-token tile stores W rows of 64 words.
__host__ __device__ inline size_t tile_word(size_t plane, int capacity, int t, int w, int W) {
  return ((plane * (size_t)(capacity >> 6) + (size_t)(t >> 6)) * (size_t)W + (size_t)w) * 64 +
         (size_t)(t & 63);
}

}  // namespace octo
