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
// Launches on one stream:
//   1. rotate_rows (x2): k_cur, v_cur -> fp16 rotated rows (coordinates in
//      part order for tensors in the OCTOPUS codec, see part_pos), which
//      every workgroup of a plane reads
//   2. chunk_attn: each wavefront rotates its own query rows, then fp16 MFMA
//      flash attention (fp32 accumulation, online softmax) whose threads
//      decode the cached window tile by tile from the packed records into
//      LDS; epilogue 1/l and R_v^T; XCD-aware workgroup order.  With split
//      tails each workgroup of a plane also takes the plane's leftover query
//      blocks over a share of the tiles and writes partials: in the first
//      pass, on the wavefronts that do not decode, for one or two leftover
//      blocks; in a second pass over the share for three or four.
//   3. chunk_tail_merge (split tails only): the leftover blocks' partials
//      merged, 1/l and R_v^T.
// The cached window is never written out: each query tile reads its packed
// records (a few bytes a coordinate) and decodes them on chip.
#include <math.h>

#include <algorithm>
#include <cstring>
#include <type_traits>

#include "octo_internal.h"

namespace octo {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr float kInvSqrtD = 0.08838834764831845f;
constexpr float kLog2e = 1.4426950408889634f;

// Order of the head coordinates in the attention tiles when a tensor uses
// the OCTOPUS codec.  A 128-coordinate row is four parts of 32 halves; part
// p holds coordinates 30 p .. 30 p + 29 (its ten whole triplets 10 p .. 10 p
// + 9, Sec. 3.2) and then coordinates 120 + 2 p and 121 + 2 p (two of the
// last eight, which belong to triplets 40..42).  One thread decodes one
// part of a row and stores it as four 16-byte chunks.  Scores and the
// weighted sum of values are sums over coordinates, so the queries and
// current keys (values) stored in the same order give the same results;
// the output is put back into coordinate order at the end.
__host__ __device__ inline int part_pos(int c) {
  return c < 120 ? 32 * (c / 30) + c % 30 : 32 * ((c - 120) >> 1) + 30 + ((c - 120) & 1);
}
__host__ __device__ inline int part_coord(int pos) {
  const int p = pos >> 5, o = pos & 31;
  return o < 30 ? 30 * p + o : 120 + 2 * p + (o - 30);
}

// ---------------------------------------------------------------- pre-pass
// Rows t < T_out of a plane of the current chunk's keys or values:
// fp16(H diag(s) x_t / sqrt(d)), zero for t >= T (tile padding).  Row t of
// an [out_rows][stride] plane (stride >= 128 halves; the halves past 128 are
// not written), coordinates in part order (part_pos) when `perm` is set.
// One workgroup takes 64 rows, sixteen lanes a row for the transform; the
// part order is applied through LDS so that each lane still stores 16 bytes.
// Every workgroup of a plane reads these rows, so they are transformed once
// here; the queries are transformed inside the attention kernel.
struct RotJob {
  const uint16_t* in;            // [planes][T][128] bf16
  int T, T_out;
  uint64_t seed;
  _Float16* out;
  int out_rows, stride;
  int tiles, planes;             // 64-row tiles per plane; planes (0: no job)
  int perm;                      // coordinates in part order
};

constexpr int kRotRow = kHeadDim + 8;   // halves per row of the LDS staging tile

__device__ inline void rotate_rows(const RotJob& jb, int tile_x, int plane, _Float16* tile) {
  typedef _Float16 half8v __attribute__((ext_vector_type(8)));
  const uint16_t* __restrict__ in = jb.in;
  _Float16* __restrict__ out = jb.out;
  const int T = jb.T, T_out = jb.T_out, out_rows = jb.out_rows;
  const uint64_t seed = jb.seed;
  // Sixteen lanes take a row, lane cl holding coordinates 8 cl .. 8 cl + 7
  // (one 16-byte load and store); a wavefront instruction covers 4 rows.
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int sub = lane >> 4, cl = lane & 15;
  const int t0 = tile_x * 64;
  float sg[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) sg[e] = splitmix_sign(seed, 8 * cl + e);
  // the wavefront's 16 rows: every load in flight at once (rows past T read
  // row T - 1 and are zeroed; with T = 0 there is nothing to read)
  uint4 raw[4] = {};
  if (T > 0) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int t = min(t0 + 16 * wave + 4 * j + sub, T - 1);
      raw[j] = *reinterpret_cast<const uint4*>(in + ((size_t)plane * T + t) * kHeadDim + 8 * cl);
    }
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int k = 16 * wave + 4 * j + sub, t = t0 + k;
    const uint32_t w[4] = {raw[j].x, raw[j].y, raw[j].z, raw[j].w};
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t h = (e & 1) ? (w[e >> 1] & 0xffff0000u) : (w[e >> 1] << 16);   // bf16 -> fp32
      v[e] = t < T ? __uint_as_float(h) * sg[e] : 0.0f;
    }
    // H (Sylvester order, unnormalized) on the row: coordinate bits 0..2
    // within the lane, bits 3..6 across the row's 16 lanes
#pragma unroll
    for (int m = 1; m < 8; m <<= 1)
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (!(e & m)) {
          const float x = v[e], y = v[e | m];
          v[e] = x + y;
          v[e | m] = x - y;
        }
#pragma unroll
    for (int m = 1; m < 16; m <<= 1) {
      const float sgm = (cl & m) ? -1.0f : 1.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = xbfly(v[e], lane_xor(v[e], m), sgm);
    }
    half8v o;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = (_Float16)(v[e] * kInvSqrtD);
    if (jb.perm) {                                  // uniform branch
      // through the wavefront's own rows of the LDS tile
#pragma unroll
      for (int e = 0; e < 8; ++e) tile[k * kRotRow + part_pos(8 * cl + e)] = o[e];
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      o = *reinterpret_cast<const half8v*>(&tile[k * kRotRow + 8 * cl]);
    }
    if (t < T_out)
      *reinterpret_cast<half8v*>(out + ((size_t)plane * out_rows + t) * jb.stride + 8 * cl) = o;
  }
}

// The two row transforms of a chunk call (current keys; current values) in
// one launch, so that the loads of one overlap the stores of the other:
// workgroups [0, n0) take job 0, the rest job 1, where n0 = tiles_0 planes_0.
__global__ __launch_bounds__(256) void rotate_rows_kernel(RotJob k, RotJob v) {
  __shared__ __attribute__((aligned(16))) _Float16 tile[64 * kRotRow];
  const int n0 = k.tiles * k.planes;
  const int id = blockIdx.x;
  if (id < n0)
    rotate_rows(k, id % k.tiles, id / k.tiles, tile);
  else
    rotate_rows(v, (id - n0) % v.tiles, (id - n0) / v.tiles, tile);
}

// Query features of the Jensen-bias correction: kFeat fp16 slots per query
// row; slot j < 128 / g holds feat_c ||(R q)_j||^2 over group j of the
// rotated coordinates, the other slots 0.
constexpr int kFeat = 8;           // feature slots per row: groups of g >= 16

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

// ---------------------------------------------------------------- attention
// The cached window is reconstructed inside the attention kernel, one 32-key
// tile at a time, into the LDS tiles the matrix cores read (OCTOPUS paper,
// Sec. 3.6: the factorized score needs u^ and gamma, never K^ in memory).
// Each thread loads the packed words of one part of one cached row (keys and
// values alike) straight into registers and writes that part as four
// 16-byte chunks:
//   - key and value rows: fp16 gamma rho^ n^ (OCTOPUS, part order) or
//     Delta^ code + z^ (group codec, coordinate order).
// The current chunk's rows come from the pre-pass (rotate_rows) by direct
// loads into the same tiles.  The value fragments of O = P V (eight keys of
// one coordinate a lane) are read from the row-major value tile with the
// transposing LDS read.
constexpr int kRG = 2;          // 16-query row groups per wavefront
constexpr int kQB = 16 * kRG;   // queries of a wavefront (one query block)
constexpr int kCWaves = 8;      // one workgroup a compute unit, two wavefronts a SIMD
constexpr int kCThreads = 64 * kCWaves;
constexpr int kSlots = 2;       // (batch, KV head) planes a workgroup may span
constexpr int kXcds = 8;        // workgroups are dealt round-robin to the XCDs
constexpr float kLazyLog2 = 8.0f;   // slack of the lazy running maximum (log2 units)
constexpr int kBN = 32;         // keys per tile
constexpr int kCurPad = kBN;    // the current rows are padded to whole tiles
// Key tile: 32 rows of 256 bytes, unpadded; 16-byte chunk c of row r is
// stored at chunk c ^ (r mod 16), so that the 8 rows one fragment read (or
// one chunk store) serves at a time fall in 8 different bank quads.
constexpr int kKChunks = kHeadDim / 8;
constexpr int kKTileBytes = kBN * kHeadDim * 2;
constexpr int kKTileInsts = kBN * kKChunks / 64;    // 64-lane direct loads of a key tile
// Value tile: 32 rows of 288 bytes (256 of values, 32 of pad), so that the
// four rows one transposing read serves at a time start 8 banks apart.
// The current values come in rows of the same length.
constexpr int kVRowBytes = 288;
constexpr int kVRowChunks = kVRowBytes / 16;
constexpr int kVSrcBytes = kHeadDim * 2;   // a value row in the workspace (unpadded)
constexpr int kVTileBytes = kBN * kVRowBytes;
constexpr int kVTileChunks = kVTileBytes / 16;
constexpr int kVTileInsts = kVTileChunks / 64;      // 64-lane direct loads of a value tile
static_assert(kVTileChunks % 64 == 0, "value tile in whole direct loads");
// A slot's two key tiles, then its two value tiles (tile u in buffer u % 2).
constexpr int kSlotBytes = 2 * kKTileBytes + 2 * kVTileBytes;
constexpr int kTilesBytes = kSlots * kSlotBytes;
// Output blocks of 16 value coordinates.
constexpr int kOB = kHeadDim / 16;
// Fourth word of a raw buffer descriptor: 32-bit data format, no swizzle.
constexpr int kBufferWord3 = 0x00020000;
// s_waitcnt immediate waiting until no vector-memory operation of the
// wavefront is outstanding (vmcnt 0; expcnt and lgkmcnt not waited for).
constexpr int kWaitVm0 = (0x7 << 4) | (0xF << 8);
// Byte offset past any buffer: a load there returns zero.
constexpr uint32_t kOutOfRange = 0x80000000u;

typedef _Float16 fp16x2 __attribute__((ext_vector_type(2)));
typedef short short4v __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
__device__ inline uint32_t pk2(fp16x2 h) { return __builtin_bit_cast(uint32_t, h); }
__device__ inline fp16x2 upk2(uint32_t u) { return __builtin_bit_cast(fp16x2, u); }
// (fp16(a), fp16(b)) rounded to nearest even, as one word
__device__ inline uint32_t pack_rne(float a, float b) {
  return __builtin_bit_cast(uint32_t, fp16x2{(_Float16)a, (_Float16)b});
}
// low halves of e0, e1 as (e0.lo, e1.lo)
__device__ inline uint32_t pair_lo(uint32_t e0, uint32_t e1) {
  return __builtin_amdgcn_perm(e1, e0, 0x05040100u);
}
// (e.hi of the first word, e.lo of the second): (y | z) of an entry (x|y), (z|0)
__device__ inline uint32_t hi_lo(uint32_t e_xy, uint32_t e_z) {
  return __builtin_amdgcn_perm(e_z, e_xy, 0x05040302u);
}
__device__ inline uint32_t mul2(uint32_t a, uint32_t b) { return pk2(upk2(a) * upk2(b)); }
// A value the compiler must treat as unknown: keeps a table index in its own
// register, so that its address is one shift-add from it.
__device__ inline uint32_t opaque(uint32_t v) {
  asm("" : "+v"(v));
  return v;
}

// One packed tensor as the attention kernel reads it.  The OCTOPUS table is
// "pre-split" (fp16 rho^ n^ at rho index K^2 + code pair, the triplet's field
// as stored) when it has at most kMaxPre entries, else it holds fp16 n^ per
// code pair with the (rho^, rho^) pairs beside it.
constexpr int kMaxPre = 512;
struct ChunkCodec {
  int sel;          // OCTOPUS: 10 b_dir + b_nrm; group: 1000 + 100 b + g
  int W;            // record words
  int tab;          // byte offset of its table in the dynamic LDS (OCTOPUS)
  int rho;          // byte offset of its rho pairs
};

struct ChunkArgs {
  const uint16_t* q;     // [B][Hq][Tq][128] bf16, rotated in the kernel
  uint64_t kseed;        // R of the keys (the queries' rotation)
  float q_post;          // scale log2(e) / sqrt(d)
  int kperm;             // queries in part order (OCTOPUS keys)
  float feat_c;          // Jensen-bias correction: query feature factor
  int feat_gs;           // ... and group size
  const _Float16* kc;    // current keys [B][Hkv][Tc_pad][128] rotated
  const _Float16* vc;    // current values [B][Hkv][Tc_pad][128] rotated
  float* out;            // [B][Hq][Tq][128]
  int Hq, Hkv, Tq;
  // 32-query blocks: qb a (batch, query head), n_blocks in all, in (batch,
  // head, block) order.  packed: workgroup w takes blocks 8 w .. 8 w + 7
  // (at most two KV planes, as a plane has bpp >= 8 blocks); else it takes
  // the bpp < 8 blocks of plane w.
  int qb, n_blocks, bpp, packed;
  // Split tails (packed mode variant): a plane's bpp = 8 upp + r blocks go to
  // upp workgroups of 8 whole blocks each, and the r leftover blocks are
  // split by keys: workgroup k of the plane also scans tiles [k tt, (k+1) tt)
  // for them and writes unnormalized partials that a second launch merges.
  // No workgroup then spans two planes.  With r <= 2 (fold) the leftover
  // blocks ride in the first pass: their 16-query row groups are taken by
  // the wavefronts that do not decode (4 .. 7), each on every nsub-th tile of
  // the share (nsub = 4 / (2 r)), giving upp nsub partials a row; otherwise a
  // second pass over the share takes them, one wavefront a block.
  int tail, upp, tail_r, tail_tt, fold, nsub;
  float* tail_o;         // [planes][r][upp nsub][32 rows][128] value sums (part order)
  float2* tail_ml;       // [planes][r][upp nsub][32 rows] (running maximum, normalizer)
  int cached, Tc, Tc_pad, capacity;
  uint64_t vseed;
  const uint32_t *k_idx, *v_idx;
  const float *k_gamma, *v_gamma;
  ChunkCodec kcod, vcod;
  int vperm;             // value rows in part order (OCTOPUS values)
  int share_tab;         // K and V use one table (same split, same codebooks)
  Codebook kcb, vcb;
};

// ---- tables
// Each table is stored in C = tab_copies(b_dir, b_nrm) interleaved copies,
// entry e of copy c at 8-byte slot C e + c, and lane L reads copy L mod C.
// With 32 copies the two banks a lane's 8-byte read touches depend on the
// lane alone, so the gathers of a wavefront (random entries) never
// conflict; tables too large for 32 copies in 32 KB get fewer.
__host__ __device__ constexpr int pre_entries(int bd, int bn) {
  return (1 << (2 * bd)) * (1 << bn) <= kMaxPre ? (1 << (2 * bd)) * (1 << bn) : (1 << (2 * bd));
}
__host__ __device__ constexpr int tab_copies(int bd, int bn) {
  return 32768 / (8 * pre_entries(bd, bn)) >= 32 ? 32 : 32768 / (8 * pre_entries(bd, bn));
}
template <int BD, int BN>
__device__ __forceinline__ void build_octo_table(const float* cx, const float* cr, char* dyn,
                                                 const ChunkCodec& c, int tid) {
  constexpr int K = 1 << BD, KK = K * K, R = 1 << BN;
  constexpr bool PRE = KK * R <= kMaxPre;
  constexpr int C = tab_copies(BD, BN);
  uint2* tab = reinterpret_cast<uint2*>(dyn + c.tab);
  for (int i = tid; i < KK * C; i += kCThreads) {
    const int e = i / C;
    const float4 n = oct_dir(cx[e % K], cx[e / K]);          // field: xi | eta << b_dir
    if (PRE) {
#pragma unroll
      for (int r = 0; r < R; ++r)
        tab[(r * KK + e) * C + i % C] =
            make_uint2(pack_rne(cr[r] * n.x, cr[r] * n.y), pack_rne(cr[r] * n.z, 0.0f));
    } else {
      tab[i] = make_uint2(pack_rne(n.x, n.y), pack_rne(n.z, 0.0f));
    }
  }
  if (!PRE && tid < R) reinterpret_cast<uint32_t*>(dyn + c.rho)[tid] = pack_rne(cr[tid], cr[tid]);
}

// ---- the packed words a thread decodes
// Thread (k = L mod 32, part pg = 2 (L / 32) + wavefront) decodes part pg of
// row k of the tile, of the keys and then of the values: OCTOPUS rows, the
// triplets 10 pg .. 10 pg + 9 and the coordinates 120 + 2 pg, 121 + 2 pg of
// triplets 40..42 (part_pos); group rows, coordinates 32 pg .. 32 pg + 31.
// A word row (word w of the 64 tokens of a tile-64 block) is 256 bytes; the
// tile's 32 tokens start at byte 4 (t0 mod 64) of it.
// Words holding the fields of triplets 10 p .. 10 p + 9 of any part p.
constexpr int main_words(int bt) {
  int m = 0;
  for (int p = 0; p < 4; ++p) {
    const int n = ((10 * bt * p) % 32 + 10 * bt + 31) / 32;
    m = n > m ? n : m;
  }
  return m;
}
// Words holding the fields of triplets 40..42.
constexpr int tail_words(int bt) { return ((43 * bt - 1) >> 5) - ((40 * bt) >> 5) + 1; }
// Codec selectors (as in ChunkCodec::sel) and the registers of one row
// part's words; selector 0 stands for "any codec, chosen at run time".
constexpr int kOctoSel[6] = {31, 42, 53, 22, 33, 44};
constexpr int kGroupSel[6] = {1216, 1232, 1316, 1332, 1416, 1432};
constexpr int row_words(int sel) {
  if (sel == 0) {
    int m = 0;
    for (int i = 0; i < 6; ++i) {
      const int a = row_words(kOctoSel[i]), b = row_words(kGroupSel[i]);
      m = a > m ? a : m;
      m = b > m ? b : m;
    }
    return m;
  }
  if (sel < 1000) {
    const int bt = 2 * (sel / 10) + sel % 10;
    return main_words(bt) + tail_words(bt) + 1;
  }
  return (sel - 1000) / 100 + 2;
}
// Calls f(std::integral_constant<int, s>) for the codec with selector s:
// SEL itself when it is not 0, else the run-time `sel`.
template <int SEL, class F>
__device__ __forceinline__ void with_codec(int sel, F&& f) {
  if constexpr (SEL != 0) {
    f(std::integral_constant<int, SEL>{});
  } else {
    switch (sel) {
      case 31: f(std::integral_constant<int, 31>{}); break;
      case 42: f(std::integral_constant<int, 42>{}); break;
      case 53: f(std::integral_constant<int, 53>{}); break;
      case 22: f(std::integral_constant<int, 22>{}); break;
      case 33: f(std::integral_constant<int, 33>{}); break;
      case 44: f(std::integral_constant<int, 44>{}); break;
      case 1216: f(std::integral_constant<int, 1216>{}); break;
      case 1232: f(std::integral_constant<int, 1232>{}); break;
      case 1316: f(std::integral_constant<int, 1316>{}); break;
      case 1332: f(std::integral_constant<int, 1332>{}); break;
      case 1416: f(std::integral_constant<int, 1416>{}); break;
      case 1432: f(std::integral_constant<int, 1432>{}); break;
    }
  }
}

// OCTOPUS rows: the words of bits [10 pg B_tri, ...), the words of triplets
// 40..42, then gamma (zero for a key past the window, `valid` false, so that
// a masked value stays finite)
template <int BD, int BN, int N>
__device__ __forceinline__ void load_octo_row(uint32_t (&w)[N], __amdgpu_buffer_rsrc_t is,
                                              __amdgpu_buffer_rsrc_t gs, int sbase, int t0, int kk,
                                              int pg, bool valid) {
  constexpr int BT = 2 * BD + BN, NWm = main_words(BT), NWe = tail_words(BT);
  static_assert(NWm + NWe + 1 <= N, "row part words");
  const int v0 = kk * 4;
  const int vm = v0 + ((10 * BT * pg) >> 5) * 256;
#pragma unroll
  for (int i = 0; i < NWm; ++i) w[i] = __builtin_amdgcn_raw_buffer_load_b32(is, vm + 256 * i, sbase, 0);
#pragma unroll
  for (int i = 0; i < NWe; ++i)
    w[NWm + i] = __builtin_amdgcn_raw_buffer_load_b32(is, v0 + 256 * (((40 * BT) >> 5) + i), sbase, 0);
  w[NWm + NWe] = __builtin_amdgcn_raw_buffer_load_b32(gs, valid ? v0 : kOutOfRange, t0 * 4, 0);
}

// Group rows: the part's code words, its scale word and zero-point word (the
// zero-point zero for a key past the window)
template <int VB, int GS, int N>
__device__ __forceinline__ void load_group_row(uint32_t (&w)[N], __amdgpu_buffer_rsrc_t is,
                                               int sbase, int kk, int pg, bool valid) {
  static_assert(VB + 2 <= N, "row part words");
  constexpr int G = kHeadDim / GS, NG = 32 / GS, WC = VB * kHeadDim / 32;
  const int v0 = kk * 4;
#pragma unroll
  for (int i = 0; i < VB; ++i) w[i] = __builtin_amdgcn_raw_buffer_load_b32(is, v0 + 256 * (VB * pg + i), sbase, 0);
  w[VB] = __builtin_amdgcn_raw_buffer_load_b32(is, v0 + 256 * (WC + (NG * pg) / 4), sbase, 0);
  w[VB + 1] = __builtin_amdgcn_raw_buffer_load_b32(
      is, valid ? v0 + 256 * (WC + G / 4 + (NG * pg) / 2) : kOutOfRange, sbase, 0);
}

// ---- row decoders (words in registers)

// Stores a row part: 16 dwords as four 16-byte chunks at the given offsets.
__device__ inline void store_part(char* tile, const int (&cw)[4], const uint32_t (&d)[16]) {
#pragma unroll
  for (int c = 0; c < 4; ++c)
    *reinterpret_cast<u32x4*>(tile + cw[c]) = u32x4{d[4 * c], d[4 * c + 1], d[4 * c + 2], d[4 * c + 3]};
}

// OCTOPUS row part (PAR: pg = 2 hi + PAR): the ten triplets as five pairs
// of three dwords, (x|y) of the first, (z of the first | x of the second),
// (y|z) of the second; then the extra dword: part 0 (x|y) of triplet 40,
// part 1 (z of 40 | x of 41), part 2 (y|z) of 41, part 3 (x|y) of 42.
// Keys and values alike: every word times gamma (in fp16).  `tab` is the
// lane's copy of the table (entry e at tab + 8 C e).
template <int BD, int BN, int PAR, int N>
__device__ __forceinline__ void dec_octo_row(const uint32_t (&w)[N], const char* tab,
                                             const char* rhotab, char* tile, const int (&cw)[4],
                                             int hi) {
  constexpr int BT = 2 * BD + BN, NWm = main_words(BT), NWe = tail_words(BT);
  constexpr int KK = 1 << (2 * BD);
  constexpr bool PRE = KK * (1 << BN) <= kMaxPre;
  constexpr int CS = 3 + __builtin_ctz(tab_copies(BD, BN));   // log2 of 8 C
  const int pg = 2 * hi + PAR;
  const int sh = (10 * BT * pg) & 31;
  uint32_t x[NWm], xe[NWe + 1];
#pragma unroll
  for (int i = 0; i < NWm; ++i) x[i] = __builtin_amdgcn_alignbit(i + 1 < NWm ? w[i + 1] : 0u, w[i], sh);
#pragma unroll
  for (int i = 0; i < NWe; ++i) xe[i] = w[NWm + i];
  xe[NWe] = 0u;
  const uint32_t gam = w[NWm + NWe];
  const uint32_t* rhop = reinterpret_cast<const uint32_t*>(rhotab);
  auto entry = [&](uint32_t f) __attribute__((always_inline)) -> uint2 {
    if constexpr (PRE) {
      return *reinterpret_cast<const uint2*>(tab + (opaque(f) << CS));
    } else {
      const uint2 e = *reinterpret_cast<const uint2*>(tab + (opaque(f & (KK - 1)) << CS));
      const uint32_t p = rhop[opaque(f >> (2 * BD))];
      return make_uint2(mul2(e.x, p), mul2(e.y, p));
    }
  };
  uint32_t d[16];
#pragma unroll
  for (int m = 0; m < 5; ++m) {
    const uint2 e0 = entry(field<BT>(x, 2 * m * BT)), e1 = entry(field<BT>(x, (2 * m + 1) * BT));
    d[3 * m] = e0.x;
    d[3 * m + 1] = pair_lo(e0.y, e1.x);
    d[3 * m + 2] = hi_lo(e1.x, e1.y);
  }
  // triplets 40..42 at bit offsets from the first tail word
  constexpr int eb = ((40 * BT) >> 5) * 32;
  auto tail = [&](int t) __attribute__((always_inline)) { return field<BT>(xe, t * BT - eb); };
  if constexpr (PAR == 0) {          // parts 0 and 2
    const uint2 ea = entry(hi ? tail(41) : tail(40));
    d[15] = hi ? hi_lo(ea.x, ea.y) : ea.x;
  } else {                           // parts 1 and 3
    const uint2 ea = entry(hi ? tail(42) : tail(40)), eb2 = entry(tail(41));
    d[15] = hi ? ea.x : pair_lo(ea.y, eb2.x);
  }
  const uint32_t G = pack_rne(__uint_as_float(gam), __uint_as_float(gam));
#pragma unroll
  for (int i = 0; i < 16; ++i) d[i] = mul2(d[i], G);
  store_part(tile, cw, d);
}

// Group-codec scale of group j from its scale word (byte j mod 4) and
// zero-point from its zero word (half j mod 2) (an E4M3 step is exact in
// fp16; the BF16 zero-point is rounded).
__device__ inline float group_scale(uint32_t sw, int j) { return e4m3_value((sw >> (8 * (j & 3))) & 0xffu); }
__device__ inline float group_zero(uint32_t zw, int j) { return __uint_as_float(((zw >> (16 * (j & 1))) & 0xffffu) << 16); }

// (code 2d | code 2d + 1) of a VB-bit stream as fp16 integers: the two fields
// spread to the halves by one multiply, over 1024 + value as fp16 bits, less
// 1024 (k1024 holds the fp16 pair (1024, 1024)).
template <int VB>
__device__ inline uint32_t code_pair(uint32_t x2, uint32_t k1024) {
  constexpr uint32_t M = (1u << VB) - 1u;
  const uint32_t y = x2 * (1u + (1u << (16 - VB)));
  return pk2(upk2((y & (M | (M << 16))) | 0x64006400u) - upk2(k1024));
}

// Group row part: the 16 words (Delta^ code + z^) of coordinates 32 pg .. 32
// pg + 31.  Keys with CORR: also the key features Delta^2 / 16 of the
// part's groups (zero in the unused slots).
template <int VB, int GS, bool CORR, bool VAL, int N>
__device__ __forceinline__ void dec_group_row(const uint32_t (&w)[N], char* tile,
                                              const int (&cw)[4], _Float16* kf, int kk,
                                              int pg, uint32_t k1024) {
  constexpr int G = kHeadDim / GS, NG = 32 / GS > 0 ? 32 / GS : 1;
  uint32_t sc[NG], zz[NG];
#pragma unroll
  for (int gi = 0; gi < NG; ++gi) {
    const int j = NG * pg + gi;
    const float dh = group_scale(w[VB], j), zf = group_zero(w[VB + 1], j);
    sc[gi] = pack_rne(dh, dh);
    zz[gi] = pack_rne(zf, zf);
    if (!VAL && CORR) kf[kk * kFeat + j] = (_Float16)(dh * dh * 0.0625f);
  }
  if (!VAL && CORR && G == 4) kf[kk * kFeat + 4 + pg] = (_Float16)0.0f;
  uint32_t cwd[VB + 1];
#pragma unroll
  for (int i = 0; i < VB; ++i) cwd[i] = w[i];
  cwd[VB] = 0u;
  uint32_t d[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const uint32_t x2 = field<2 * VB>(cwd, 2 * i * VB);
    const int gi = (2 * i) / GS;
    d[i] = pk2(__builtin_elementwise_fma(upk2(code_pair<VB>(x2, k1024)), upk2(sc[gi]), upk2(zz[gi])));
  }
  store_part(tile, cw, d);
}

// Workgroup barrier for the tile pipeline: this wave's LDS operations are
// complete, its global loads stay in flight (the pipeline waits for its
// direct-to-LDS loads itself, before the barrier that publishes them).  The
// memory clobber keeps the compiler from moving memory accesses across it.
__device__ inline void tile_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Lane layout of v_mfma_f32_16x16x32_f16 (wave of 64, L = lane):
//   A[i][k]: i = L % 16, k = 8 (L / 16) + e  (e = element 0..7)
//   B[k][j]: j = L % 16, k = 8 (L / 16) + e
//   D[i][j]: i = 4 (L / 16) + r, j = L % 16  (r = register 0..3)
// Scores are computed transposed, S^T = K Q^T (keys are rows), so that each
// lane ends up with 4 keys of one query, which is exactly the A operand
// layout P needs for O = P V with keys as the contraction index: slot e of
// lane group g is key 16 (e / 4) + 4 g + e % 4.  Each wavefront owns two
// 16-query row groups, so every key / value fragment read from LDS feeds two
// MFMAs.  The softmax state is updated once per tile.
//
// Value fragments: the transposing read (ds_read_b64_tr_b16) gives lane i of
// a 16-lane group, element j, element i % 4 of the four halves that lane
// 4 j + i / 4 of the group addressed.  Lane s = 4 j + q of group g
// addresses row 4 g + j (then 16 + 4 g + j) of the value tile at
// coordinates 16 c + 4 q .. 16 c + 4 q + 3, so lane i receives coordinate
// 16 c + i of keys 4 g + j (then 16 + 4 g + j): its B fragment.
//
// Workgroups: a wavefront takes one block of 32 queries of one (batch,
// query head) and every key of its plane; a workgroup takes eight
// consecutive blocks, which may end one plane and begin the next (two
// "slots", each with its own tiles).  The threads decode each cached tile
// once for every wavefront of its plane: wavefront w decodes slot w / 4,
// keys (w / 2 even) or values, part 2 (L / 32) + w % 2 of row L % 32 -- one
// row part a thread a tile.  With a workgroup a compute unit the LDS holds
// the tables in 32 lane-private copies (see tab_copies).
//
// Tiles: the cached window's ceil(cached / 32) tiles first, then the current
// chunk's; tile u lives in buffer u % 2 of its slot.  Iteration t: the words
// of cached tile t + 2 are requested (registers of stage t % 2), or the rows
// of current tile t + 1 (direct loads into buffer (t + 1) % 2); tile t is
// computed; the threads decode cached tile t + 1 (words of stage (t + 1) %
// 2) into buffer (t + 1) % 2; one barrier.  The loop is unrolled by two so
// that buffer offsets and word stages are constants.
//
// XCD-aware order: the hardware deals consecutive workgroup ids to the 8
// XCDs in turn, so the linear id is mapped such that consecutive workgroups
// (the query blocks of one plane) run on the same XCD and stream its keys
// and values through that XCD's L2 together.
//
// CORR: the Jensen-bias correction ("Quantized Keys Steal Attention",
// Eq. 15).  Its bias is a rank-(128 / g) product of query and key features,
// so it is one more k-slice of the score MFMA per 16 cached keys, whose slots
// 0..7 (lane group 0) hold the features and the rest zeros.
template <bool CORR, int KSEL, int VSEL>
__global__ __launch_bounds__(kCThreads, 1) void chunk_attn_kernel(ChunkArgs a) {
  static_assert(KSEL == VSEL, "one codec for both tensors, or chosen at run time");
  constexpr int NW = row_words(KSEL);
  __shared__ __attribute__((aligned(1024))) char tiles[kTilesBytes];
  __shared__ __attribute__((aligned(16))) _Float16 kfs[kSlots][2][CORR ? kBN * kFeat : 8];
  __shared__ __attribute__((aligned(16))) _Float16 qfs[CORR ? (kCWaves * kQB + 64) * kFeat : 8];
  extern __shared__ __attribute__((aligned(16))) char dyn[];

  const int tid = threadIdx.x, L = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = L & 15, grp = L >> 4;
  const int n_units = gridDim.x;
  const int id = blockIdx.x;
  // id -> (xcd, local); units are split into 8 contiguous ranges, range x
  // running on XCD x.
  const int per_xcd = (n_units + kXcds - 1) / kXcds;
  const int xcd = id % kXcds, local = id / kXcds;
  const int full_xcds = n_units - (per_xcd - 1) * kXcds;   // XCDs with per_xcd units
  const int unit = xcd < full_xcds ? xcd * per_xcd + local
                                   : full_xcds * per_xcd + (xcd - full_xcds) * (per_xcd - 1) + local;
  // the workgroup's query blocks [start, start + count) and their planes
  const int start = a.tail ? (unit / a.upp) * a.bpp + (unit % a.upp) * kCWaves
                           : (a.packed ? unit * kCWaves : unit * a.bpp);
  const int count = a.tail ? kCWaves : (a.packed ? min(kCWaves, a.n_blocks - start) : a.bpp);
  const int gq = a.Hq / a.Hkv;
  auto plane_of = [&](int g) {
    const int bhq = g / a.qb;
    return (bhq / a.Hq) * a.Hkv + (bhq % a.Hq) / gq;
  };
  const int plane0 = plane_of(start), plane1 = plane_of(start + count - 1);
  const bool two = plane1 != plane0;
  // this wavefront's block (batch b, query head hq, queries q0 ..) and slot
  // (the first pass; a split tail's pass takes a leftover block)
  bool active = wave < count;
  int gb = start + min(wave, count - 1);
  int bh = gb / a.qb, q0 = (gb % a.qb) * kQB;
  int cslot = plane_of(gb) != plane0;
  // its decode task: slot, tensor (0 keys, 1 values), part parity
  const int dslot = wave >> 2, dten = (wave >> 1) & 1, dpar = wave & 1;
  const bool dact = dslot == 0 || two;
  const size_t dplane = dslot ? plane1 : plane0;
  const int dsel = dten ? a.vcod.sel : a.kcod.sel;
  const int dW = dten ? a.vcod.W : a.kcod.W;
  const int dtab = dten ? a.vcod.tab : a.kcod.tab, drho = dten ? a.vcod.rho : a.kcod.rho;

  // ---- codebooks to LDS (at the end of the tile area: buffer 1 of slot 1,
  // first written after the barriers of tile 0), one value a lane from the
  // argument block; then the tables
  constexpr int kCb = kMaxXi + kMaxRho;
  float* cbs = reinterpret_cast<float*>(tiles + kTilesBytes) - 2 * kCb;
  static_assert(kCWaves * kQB * kHeadDim * 2 + 2 * kCb * 4 <= kTilesBytes,
                "the query stagings and the codebooks share the tile area");
  {
    // constant indices into the argument block (a run-time index would put
    // a copy of it in private memory)
    float ck = 0.0f, cv = 0.0f;
#pragma unroll
    for (int i = 0; i < kCb; ++i) {
      ck = tid == i ? (i < kMaxXi ? a.kcb.xi[i] : a.kcb.rho[i - kMaxXi]) : ck;
      cv = tid == i ? (i < kMaxXi ? a.vcb.xi[i] : a.vcb.rho[i - kMaxXi]) : cv;
    }
    if (tid < kCb) {
      cbs[tid] = ck;
      cbs[kCb + tid] = cv;
    }
  }
  // ---- the wavefront's 32 query rows (rows past Tq repeat the last):
  // fp16(post H diag(s) q) in part order for OCTOPUS keys, staged in the
  // wavefront's 8 KB of the tile area (free until the first tile; the
  // codebooks sit past the eight stagings) with 16-byte chunk c of row r at
  // chunk c ^ (r mod 16), then read back as the B fragments.  Sixteen lanes
  // take a row, lane cl coordinates 8 cl .. 8 cl + 7: butterflies over bits
  // 0..2 in registers, 3..6 across the row's lanes.  With the correction the
  // group sums of the squared rotated coordinates give the query features.
  half8 qf[kRG][4];
  // Stages 16 RG query rows q0_ .. of (batch, head) bh_ and reads back their
  // fragments into dst; with the correction their features go to rows
  // frow .. of qfs.
  auto stage = [&](int bh_, int q0_, auto& dst, int frow) __attribute__((always_inline)) {
    constexpr int RG = std::extent<std::remove_reference_t<decltype(dst)>>::value;
    _Float16* stg = reinterpret_cast<_Float16*>(tiles) + wave * kQB * kHeadDim;
    // from an opaque copy of the lane index, so that a later call forms its
    // signs and offsets afresh instead of keeping the first call's live
    int lq = L;
    asm volatile("" : "+v"(lq));
    const int sub = lq >> 4, cl = lq & 15;
    float sg[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) sg[e] = splitmix_sign(a.kseed, 8 * cl + e);
    uint4 raw[4 * RG];
#pragma unroll
    for (int j = 0; j < 4 * RG; ++j) {
      const int qrow = min(q0_ + 4 * j + sub, a.Tq - 1);
      raw[j] = *reinterpret_cast<const uint4*>(a.q + ((size_t)bh_ * a.Tq + qrow) * kHeadDim + 8 * cl);
    }
#pragma unroll
    for (int j = 0; j < 4 * RG; ++j) {
      const int r = 4 * j + sub;
      const uint32_t w[4] = {raw[j].x, raw[j].y, raw[j].z, raw[j].w};
      float v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e)
        v[e] = __uint_as_float((e & 1) ? (w[e >> 1] & 0xffff0000u) : (w[e >> 1] << 16)) * sg[e];
#pragma unroll
      for (int m = 1; m < 8; m <<= 1)
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (!(e & m)) {
            const float x = v[e], y = v[e | m];
            v[e] = x + y;
            v[e | m] = x - y;
          }
#pragma unroll
      for (int m = 1; m < 16; m <<= 1) {
        const float sgm = (cl & m) ? -1.0f : 1.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = xbfly(v[e], lane_xor(v[e], m), sgm);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int pos = a.kperm ? part_pos(8 * cl + e) : 8 * cl + e;
        stg[r * kHeadDim + ((((pos >> 3) ^ (r & 15)) << 3) | (pos & 7))] = (_Float16)(v[e] * a.q_post);
      }
      if constexpr (CORR) {
        float sq = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) sq = fmaf(v[e] * kInvSqrtD, v[e] * kInvSqrtD, sq);
        const int lpg = a.feat_gs / 8;                 // lanes of a group
        for (int m = 1; m < lpg; m <<= 1) sq += __shfl_xor(sq, m, 64);
        const int ng = kHeadDim / a.feat_gs;
        const float f = __shfl(sq, 16 * sub + min(cl, ng - 1) * lpg, 64);
        if (cl < kFeat) qfs[(frow + r) * kFeat + cl] = (_Float16)(cl < ng ? a.feat_c * f : 0.0f);
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // query 16 rg + col, dims 32 s + 8 grp + e: chunk 4 s + grp of its row
    const int qcol = lq & 15, qgrp = lq >> 4;
#pragma unroll
    for (int rg = 0; rg < RG; ++rg)
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4)
        dst[rg][s4] = *reinterpret_cast<const half8*>(
            stg + (16 * rg + qcol) * kHeadDim + (((4 * s4 + qgrp) ^ qcol) << 3));
  };
  stage(bh, q0, qf, wave * kQB);
  // fold mode: wavefront 4 + xw (which does not decode) also takes row group
  // xrg of leftover block xj on tiles xsub, xsub + nsub, .. of the
  // workgroup's share (its query features in rows 256 + 16 xw .. of qfs)
  const int xw = wave - 4, x2r = 2 * max(a.tail_r, 1);
  const bool xact = a.fold && xw >= 0;
  const int xg = xact ? xw % x2r : 0, xj = xg >> 1, xrg = xg & 1, xsub = xact ? xw / x2r : 0;
  half8 qx[1][4];
  if (xact) {
    const int gbx = plane0 * a.bpp + kCWaves * a.upp + xj;
    stage(gbx / a.qb, (gbx % a.qb) * kQB + 16 * xrg, qx, kCWaves * kQB + 16 * xw);
  }
  __syncthreads();                     // the stagings are read before tile 0 lands
  {
    const float *cxk = cbs, *crk = cbs + kMaxXi, *cxv = cbs + kCb, *crv = cbs + kCb + kMaxXi;
    with_codec<KSEL>(a.kcod.sel, [&](auto cs) __attribute__((always_inline)) {
      constexpr int C = decltype(cs)::value;
      if constexpr (C < 1000) build_octo_table<C / 10, C % 10>(cxk, crk, dyn, a.kcod, tid);
    });
    if (!a.share_tab) {
      with_codec<VSEL>(a.vcod.sel, [&](auto cs) __attribute__((always_inline)) {
        constexpr int C = decltype(cs)::value;
        if constexpr (C < 1000) build_octo_table<C / 10, C % 10>(cxv, crv, dyn, a.vcod, tid);
      });
    }
  }
  // ---- passes: the workgroup's blocks over every tile; then, for a split
  // tail, the plane's leftover blocks over this workgroup's share of tiles.
  // Each pass forms its per-thread offsets afresh, so that none is kept
  // live through the other's epilogue.
  auto run_pass = [&](auto pass_c) __attribute__((always_inline)) {
  constexpr int pass = decltype(pass_c)::value;
  // fp16 pair (1024, 1024) in a register (for the group codec's integers)
  uint32_t k1024;
  asm volatile("v_mov_b32 %0, 0x64006400" : "=v"(k1024));

  // ---- per-thread constants of the decoder: the byte offsets (buffer 0 of
  // the task's slot) of the four chunks of the thread's row part
  int tw[4];
  {
    const int kk = L & 31, pg = 2 * (L >> 5) + dpar, base = dslot * kSlotBytes;
#pragma unroll
    for (int d = 0; d < 4; ++d)
      tw[d] = base + (dten ? 2 * kKTileBytes + kk * kVRowBytes + 64 * pg + 16 * d
                           : kk * 256 + (((4 * pg + d) ^ (kk & 15)) << 4));
  }
  const int tstage = dten ? kVTileBytes : kKTileBytes;   // buffer 1 less buffer 0

  floatx4 o[kRG][kOB];
  // nm: minus the running maximum of query q0 + 16 rg + col in all four
  // slots (log2 units; 0 until the first tile of the pass sets it), the
  // initial value of the tile's score products; ls: the normalizers of
  // queries q0 + 16 rg + 4 grp + r, summed by the products P 1
  floatx4 nm[kRG], ls[kRG];

  // the task's packed stream and gammas, and the current chunk's rows of the
  // task's plane (loads past a plane's range return zero)
  const int tiles64 = a.capacity >> 6;
  const bool dgroup = dsel >= 1000;
  const __amdgpu_buffer_rsrc_t dis = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint32_t*>((dten ? a.v_idx : a.k_idx) + dplane * tiles64 * dW * 64), (short)0,
      a.capacity * dW * 4, kBufferWord3);
  const __amdgpu_buffer_rsrc_t dgs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(dgroup ? nullptr : (dten ? a.v_gamma : a.k_gamma) + dplane * a.capacity),
      (short)0, dgroup ? 0 : a.capacity * 4, kBufferWord3);
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<_Float16*>(a.kc + dplane * a.Tc_pad * kHeadDim), (short)0,
      a.Tc_pad * kHeadDim * 2, kBufferWord3);
  const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<_Float16*>(a.vc + dplane * a.Tc_pad * kHeadDim), (short)0,
      a.Tc_pad * kVSrcBytes, kBufferWord3);

  const int n_ct = (a.cached + kBN - 1) / kBN, n_rt = (a.Tc + kBN - 1) / kBN;
  const int n_tiles = n_ct + n_rt;
  int t_lo = 0, t_hi = n_tiles;        // the tiles of the current pass
  // a split tail's pass: leftover block tj of the plane is taken by
  // wavefront 4 + tj, so that the wavefronts that compute (4 ..) and those
  // that decode (0 .. 3) differ and a tile's products overlap the next
  // tile's decoding
  const int tj = wave - 4;
  if constexpr (pass == 1) {
    const int k = unit % a.upp;
    t_lo = min(n_tiles, k * a.tail_tt);
    t_hi = min(n_tiles, t_lo + a.tail_tt);
    active = tj >= 0 && tj < a.tail_r;
    gb = plane0 * a.bpp + kCWaves * a.upp + min(max(tj, 0), a.tail_r - 1);
    bh = gb / a.qb;
    q0 = (gb % a.qb) * kQB;
    cslot = 0;
    __syncthreads();                   // the first pass's epilogue rows are read
    stage(bh, q0, qf, wave * kQB);
    __syncthreads();
  }
#pragma unroll
  for (int rg = 0; rg < kRG; ++rg) {
#pragma unroll
    for (int c = 0; c < kOB; ++c) o[rg][c] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
    nm[rg] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
    ls[rg] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
  }


  // Words of the thread's row part of cached tile u into registers.
  auto load_words = [&](int u, uint32_t (&w)[NW]) __attribute__((always_inline)) {
    const int t0 = u * kBN;
    // the per-thread offsets are formed here from an opaque copy of the
    // thread index, tile by tile, rather than kept live across the loop
    int lt = tid;
    asm volatile("" : "+v"(lt));
    const int kk = lt & 31, pg = 2 * ((lt & 63) >> 5) + dpar;
    const bool valid = kk < a.cached - t0;
    // byte offset of the tile's first token in word row 0 of a W-word plane
    const int sb = (t0 >> 6) * dW * 256 + (t0 & 63) * 4;
    with_codec<KSEL>(dsel, [&](auto cs) __attribute__((always_inline)) {
      constexpr int C = decltype(cs)::value;
      if constexpr (C < 1000) load_octo_row<C / 10, C % 10>(w, dis, dgs, sb, t0, kk, pg, valid);
      else load_group_row<(C - 1000) / 100, C % 100>(w, dis, sb, kk, pg, valid);
    });
  };
  // Decodes the thread's row part of cached tile u from its words into
  // buffer S (= u % 2) of its slot.  Keys past the window (in its ragged last
  // tile) decode from whatever words follow it: their scores are masked, and
  // their values are finite (their gammas or zero-points load as zero).
  auto decode = [&](int u, auto stage, const uint32_t (&w)[NW]) __attribute__((always_inline)) {
    constexpr int S = decltype(stage)::value;
    int lt = tid;
    asm volatile("" : "+v"(lt));
    const int kk = lt & 31, hi = (lt & 63) >> 5, pg = 2 * hi + dpar;
    char* tb = tiles + S * tstage;               // tw holds the slot's offsets
    with_codec<KSEL>(dsel, [&](auto cs) __attribute__((always_inline)) {
      constexpr int C = decltype(cs)::value;
      if constexpr (C < 1000) {
        constexpr int BD = C / 10, BN = C % 10, NC = tab_copies(BD, BN);
        const char* tab = dyn + dtab + ((lt & (NC - 1)) << 3);
        const char* rt = dyn + drho;
        if (dpar) dec_octo_row<BD, BN, 1>(w, tab, rt, tb, tw, hi);
        else dec_octo_row<BD, BN, 0>(w, tab, rt, tb, tw, hi);
      } else {
        constexpr int VB = (C - 1000) / 100, GS = C % 100;
        if (dten) dec_group_row<VB, GS, false, true>(w, tb, tw, nullptr, kk, pg, k1024);
        else dec_group_row<VB, GS, CORR, false>(w, tb, tw, kfs[dslot][S], kk, pg, k1024);
      }
    });
  };
  // Requests the rows of current tile u into buffer S (= u % 2) of the
  // thread's slot, by the slot's four wavefronts; nothing is waited for here.
  auto request_rows = [&](int u, auto stage) __attribute__((always_inline)) {
    constexpr int S = decltype(stage)::value;
    const int kt0 = (u - n_ct) * kBN;
    char* ks = tiles + dslot * kSlotBytes + S * kKTileBytes;
    char* vs = tiles + dslot * kSlotBytes + 2 * kKTileBytes + S * kVTileBytes;
    // source offsets, formed here (current tiles are few) rather than kept
    // in registers across the loop
    uint32_t lx = L;
    asm volatile("" : "+v"(lx));
    const int lw = wave & 3;
    // key tile: lane L of load j fills stored chunk p = 64 j + L, row p / 16,
    // logical chunk (p % 16) ^ (row % 16)
#pragma unroll
    for (int i = 0; i < kKTileInsts / 4; ++i) {
      const int j = 4 * i + lw;
      const uint32_t p = 64 * j + lx;
      const uint32_t kr = p / kKChunks, kc = (p % kKChunks) ^ (kr % kKChunks);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, ks + 1024 * j, 16, (kr * kHeadDim + kc * 8) * 2,
                                               kt0 * kHeadDim * 2, 0, 0);
    }
    // value tile: stored chunk p = 64 j + L is chunk p mod 18 of padded row
    // p / 18, the 16 bytes at 16 (p mod 18) of that row (256 bytes in the
    // workspace) for the first 16 chunks of a row; the two pad chunks read
    // nothing
#pragma unroll
    for (int i = 0; i < (kVTileInsts + 3) / 4; ++i) {
      const int j = 4 * i + lw;
      const uint32_t p = 64 * j + lx, vr = p / kVRowChunks, vcn = p % kVRowChunks;
      if (j < kVTileInsts)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, vs + 1024 * j, 16,
                                                 vcn < 16 ? vr * kVSrcBytes + 16 * vcn : kOutOfRange,
                                                 kt0 * kVSrcBytes, 0, 0);
    }
  };
  // per-lane offsets of the key fragments of slice s (row col, logical chunk
  // 4 s + grp, stored at chunk (4 s + grp) ^ col; row 16 kt + col adds 4096
  // kt) and of the transposing value reads (row 4 grp + col / 4, coordinates
  // 4 (col % 4) ..; the other four keys 16 rows on, block c 32 c bytes on)
  int kfr[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) kfr[s] = col * 256 + (((4 * s + grp) ^ col) << 4);
  const int vtr = (4 * grp + (col >> 2)) * kVRowBytes + 8 * (col & 3);
  // One tile from buffer S.  The first tile sets the running maxima; only
  // the ragged last tile of each segment masks keys.  (Both are uniform
  // branches on the scores alone, so that one copy of the MFMA chains
  // serves every tile.)
  auto compute = [&](int u, auto stage, bool first, auto& qfa, auto& oa, auto& nma, auto& lsa, int frow)
      __attribute__((always_inline)) {
    constexpr int S = decltype(stage)::value;
    constexpr int RG = std::extent<std::remove_reference_t<decltype(nma)>>::value;
    const bool cachedt = u < n_ct;
    const int nvalid = cachedt ? a.cached - u * kBN : a.Tc - (u - n_ct) * kBN;
    const char* ks = tiles + cslot * kSlotBytes + S * kKTileBytes;
    const char* vs = tiles + cslot * kSlotBytes + 2 * kKTileBytes + S * kVTileBytes;
    // scores of the tile's keys (log2 units): st[kt][rg][r] = key 16 kt + 4 grp + r
    floatx4 st[kBN / 16][RG];
    const half8 zero8 = {};
    if constexpr (!CORR) {
      __builtin_amdgcn_sched_barrier(0);
      half8 kf8[2][4];
#pragma unroll
      for (int kt = 0; kt < kBN / 16; ++kt)
#pragma unroll
        for (int s = 0; s < 4; ++s) kf8[kt][s] = *reinterpret_cast<const half8*>(ks + 16 * kt * 256 + kfr[s]);
#pragma unroll
      for (int kt = 0; kt < kBN / 16; ++kt) {
#pragma unroll
        for (int rg = 0; rg < RG; ++rg) st[kt][rg] = nma[rg];
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
          for (int rg = 0; rg < RG; ++rg)
            st[kt][rg] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf8[kt][s], qfa[rg][s], st[kt][rg], 0, 0, 0);
      }
      // reads of slice 0 first; then each pair of products followed by one read
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int kt = 0; kt < kBN / 16; ++kt) {
      if constexpr (CORR) {
#pragma unroll
      for (int rg = 0; rg < RG; ++rg) st[kt][rg] = nma[rg];
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const half8 kf = *reinterpret_cast<const half8*>(ks + 16 * kt * 256 + kfr[s]);
#pragma unroll
        for (int rg = 0; rg < RG; ++rg)
          st[kt][rg] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf, qfa[rg][s], st[kt][rg], 0, 0, 0);
      }
      }
      if constexpr (CORR) {
        if (cachedt) {
          // minus the Jensen bias of keys 16 kt + (0..15), in log2 units
          // (slots 8..31 of both operands are zero: lane groups 1..3 read nothing)
          half8 kf5 = zero8;
          if (grp == 0) kf5 = *reinterpret_cast<const half8*>(&kfs[cslot][S][(16 * kt + col) * kFeat]);
#pragma unroll
          for (int rg = 0; rg < RG; ++rg) {
            half8 qf5 = zero8;
            if (grp == 0)
              qf5 = *reinterpret_cast<const half8*>(&qfs[(frow + 16 * rg + col) * kFeat]);
            st[kt][rg] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf5, qf5, st[kt][rg], 0, 0, 0);
          }
        }
      }
    }
    // x = s - m in log2 units relative to the running maximum (0 before
    // the first tile): the products started from -m
    float x[RG][kBN / 4];
#pragma unroll
    for (int rg = 0; rg < RG; ++rg)
#pragma unroll
      for (int e = 0; e < kBN / 4; ++e) x[rg][e] = st[e >> 2][rg][e & 3];
    if (nvalid < kBN) {
      // keys 16 kt + 4 grp + r past the segment (an opaque lane offset, so
      // that no per-slot key index is kept in registers)
      int k4 = 4 * grp;
      asm volatile("" : "+v"(k4));
#pragma unroll
      for (int rg = 0; rg < RG; ++rg)
#pragma unroll
        for (int e = 0; e < kBN / 4; ++e)
          if (16 * (e >> 2) + k4 + (e & 3) >= nvalid) x[rg][e] = -INFINITY;
    }
    // Lazy running maximum: a row moves its maximum (and rescales its sums)
    // only when a score exceeds it by more than kLazyLog2 -- or on the first
    // tile, which sets it -- so that nearly every tile skips the rescale;
    // probabilities then stay below 2^kLazyLog2, well inside fp16, and the
    // final 1/l cancels the shift.
    float sh[RG];
    bool any = false;
#pragma unroll
    for (int rg = 0; rg < RG; ++rg) {
      float mx = x[rg][0];
#pragma unroll
      for (int e = 1; e < kBN / 4; ++e) mx = fmaxf(mx, x[rg][e]);
      mx = rows_max(mx);
      const bool up = first || mx > kLazyLog2;
      sh[rg] = up ? mx : 0.0f;
      any = any || __ballot(up) != 0;
    }
    // A rescale moves the rows' maxima, scales O and the sums by 2^-shift
    // (on the first tile, both 0 and a shift of either sign, by at most 1)
    // and shifts the scores, all in place; one chain of P V products then
    // follows either way, so that each accumulator's only reader is its
    // product and the product writes it in place.
    if (any) {
#pragma unroll
      for (int rg = 0; rg < RG; ++rg) {
#pragma unroll
        for (int r = 0; r < 4; ++r) nma[rg][r] -= sh[rg];
        // O rows and normalizers (queries q0 + 16 rg + 4 grp + r)
        const float alpha = __builtin_amdgcn_exp2f(-fmaxf(sh[rg], 0.0f));
        float al[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) al[r] = __shfl(alpha, 4 * grp + r, 64);
#pragma unroll
        for (int r = 0; r < 4; ++r) lsa[rg][r] *= al[r];
#pragma unroll
        for (int c = 0; c < kOB; ++c)
#pragma unroll
          for (int r = 0; r < 4; ++r) oa[rg][c][r] *= al[r];
#pragma unroll
        for (int e = 0; e < kBN / 4; ++e) x[rg][e] -= sh[rg];
      }
    }
    // P and its row sums (P 1, of the fp16 P that the products take), then
    // O += P V (value fragments by the transposing read)
    half8 pf[RG];
    const half8 ones = {1, 1, 1, 1, 1, 1, 1, 1};
#pragma unroll
    for (int rg = 0; rg < RG; ++rg) {
#pragma unroll
      for (int e = 0; e < kBN / 4; ++e)
        // the raw exp2 (flushing results below the normal range to zero) is
        // exact enough next to the row's largest terms (at least 1)
        pf[rg][e] = (_Float16)__builtin_amdgcn_exp2f(x[rg][e]);
      lsa[rg] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pf[rg], ones, lsa[rg], 0, 0, 0);
    }
#pragma unroll
    for (int c = 0; c < kOB; ++c) {
      typedef __attribute__((address_space(3))) short4v lds_short4;
      const short4v lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)(vs + vtr + 32 * c));
      const short4v hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_short4*)(vs + vtr + 16 * kVRowBytes + 32 * c));
      const half8 vf = __builtin_bit_cast(half8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
      for (int rg = 0; rg < RG; ++rg)
        oa[rg][c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pf[rg], vf, oa[rg][c], 0, 0, 0);
    }
  };

  // fold mode: the extra row group's share of tiles and softmax state
  int x_lo = 0, x_hi = 0;
  if (xact) {
    x_lo = min(n_tiles, (unit % a.upp) * a.tail_tt);
    x_hi = min(n_tiles, x_lo + a.tail_tt);
  }
  floatx4 ox[1][kOB], nmx[1], lsx[1];
#pragma unroll
  for (int c = 0; c < kOB; ++c) ox[0][c] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
  nmx[0] = lsx[0] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
  // ---- passes: the workgroup's blocks over every tile; then, for a split
  // tail, the plane's leftover blocks over this workgroup's share of tiles
  // ---- the tile pipeline over [t_lo, t_hi): the words of cached tile u in
  // registers of stage (u - t_lo) % 2, requested two tiles ahead
  const int c_hi = min(n_ct, t_hi);    // cached tiles of the pass end here
  uint32_t w0[NW] = {}, w1[NW] = {};
  if (dact && t_lo < c_hi) load_words(t_lo, w0);
  if (dact && t_lo + 1 < c_hi) load_words(t_lo + 1, w1);
  if (dact && t_lo >= n_ct && t_lo < t_hi) request_rows(t_lo, std::integral_constant<int, 0>{});
  lds_barrier();                       // tables built
  if (t_lo < c_hi) {
    if (dact) decode(t_lo, std::integral_constant<int, 0>{}, w0);
  } else {
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
  }
  lds_barrier();
  // iteration t, buffer and word stage S = (t - t_lo) % 2
  auto iter = [&](int t, auto stage, uint32_t (&wS)[NW], uint32_t (&wN)[NW]) __attribute__((always_inline)) {
    constexpr int S = decltype(stage)::value;
    using Next = std::integral_constant<int, 1 - S>;
    if (dact && t + 2 < c_hi) load_words(t + 2, wS);
    const bool next_cur = t + 1 >= n_ct && t + 1 < t_hi;
    if (dact && next_cur) request_rows(t + 1, Next{});
    if (active) compute(t, stage, t == t_lo, qf, o, nm, ls, wave * kQB);
    if constexpr (pass == 0) {
      if (xact && t >= x_lo && t < x_hi && ((t - x_lo) & (a.nsub - 1)) == xsub)
        compute(t, stage, t == x_lo + xsub, qx, ox, nmx, lsx, kCWaves * kQB + 16 * xw);
    }
    if (t + 1 < c_hi) {
      if (dact) decode(t + 1, Next{}, wN);
    } else if (next_cur) {
      __builtin_amdgcn_s_waitcnt(kWaitVm0);
    }
    tile_barrier();                    // tile t read by all; tile t + 1 in place
  };
  for (int t = t_lo; t < t_hi; t += 2) {
    iter(t, std::integral_constant<int, 0>{}, w0, w1);
    if (t + 1 < t_hi) iter(t + 1, std::integral_constant<int, 1>{}, w1, w0);
  }

  if constexpr (pass == 0) {
    // ---- fold mode: the extra row group's partial (rows 16 xrg .. of
    // leftover block xj; partial (unit % upp) nsub + xsub of the plane)
    if (xact) {
      const size_t row0 = (((size_t)plane0 * a.tail_r + xj) * (a.upp * a.nsub) +
                           (unit % a.upp) * a.nsub + xsub) * kQB + 16 * xrg;
      const bool any_tile = x_lo + xsub < x_hi;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float m = -__shfl(nmx[0][0], 4 * grp + r, 64);
        if (col == 0) a.tail_ml[row0 + 4 * grp + r] = make_float2(any_tile ? m : -INFINITY, lsx[0][r]);
      }
#pragma unroll
      for (int c = 0; c < kOB; ++c)
#pragma unroll
        for (int r = 0; r < 4; ++r) a.tail_o[(row0 + 4 * grp + r) * kHeadDim + 16 * c + col] = ox[0][c][r];
    }
  }
  if constexpr (pass == 1) {
    // ---- a split tail's partial: per query row of the leftover block the
    // running maximum (-inf for an empty share of tiles) and normalizer,
    // and the unnormalized value sums in part order
    if (active) {
      const size_t row0 =
          (((size_t)plane0 * a.tail_r + tj) * a.upp + unit % a.upp) * kQB;
#pragma unroll
      for (int rg = 0; rg < kRG; ++rg) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float m = -__shfl(nm[rg][0], 4 * grp + r, 64);
          if (col == 0)
            a.tail_ml[row0 + 16 * rg + 4 * grp + r] = make_float2(t_hi > t_lo ? m : -INFINITY, ls[rg][r]);
        }
#pragma unroll
        for (int c = 0; c < kOB; ++c)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            a.tail_o[(row0 + 16 * rg + 4 * grp + r) * kHeadDim + 16 * c + col] = o[rg][c][r];
      }
    }
    return;
  }
  // ---- epilogue, one 16-query row group at a time: 1/l; value columns back
  // to coordinate order (OCTOPUS values, through the wavefront's own rows of
  // LDS); then R_v^T = diag(s_v) H / sqrt(d) on every query row.  Lane holds
  // coordinate 16 c + col of queries q0 + 16 rg + 4 grp + r: the Hadamard
  // butterflies on coordinate bits 4..6 are register-local, bits 0..3 cross
  // lanes within each 16-lane group.
  if (!active) return;
  float sv[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) sv[c] = kInvSqrtD * splitmix_sign(a.vseed, 16 * c + col);
  constexpr int kORow = kHeadDim + 4;                  // floats per query row in LDS
  static_assert(kCWaves * 16 * kORow * 4 <= kTilesBytes, "epilogue rows fit the tiles");
  float* ob = reinterpret_cast<float*>(tiles) + wave * (16 * kORow);
#pragma unroll
  for (int rg = 0; rg < kRG; ++rg) {
    float v[8][4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float l = ls[rg][r];
      const float li = l > 0.0f ? 1.0f / l : 0.0f;
#pragma unroll
      for (int c = 0; c < 8; ++c) v[c][r] = o[rg][c][r] * li;
    }
    if (a.vperm) {
      // column 16 c + col holds coordinate part_coord(16 c + col)
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const int crd = part_coord(16 * c + col);
#pragma unroll
        for (int r = 0; r < 4; ++r) ob[(4 * grp + r) * kORow + crd] = v[c][r];
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
      for (int c = 0; c < 8; ++c)
#pragma unroll
        for (int r = 0; r < 4; ++r) v[c][r] = ob[(4 * grp + r) * kORow + 16 * c + col];
      // the rows are read before the next row group writes them
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
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
    for (int m = 8; m >= 1; m >>= 1) {
      const float sgm = (col & m) ? -1.0f : 1.0f;
#pragma unroll
      for (int c = 0; c < 8; ++c)
#pragma unroll
        for (int r = 0; r < 4; ++r) v[c][r] = xbfly(v[c][r], lane_xor(v[c][r], m), sgm);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int q = q0 + 16 * rg + 4 * grp + r;
      if (q >= a.Tq) continue;
      float* dst = a.out + ((size_t)bh * a.Tq + q) * kHeadDim;
#pragma unroll
      for (int c = 0; c < 8; ++c) dst[16 * c + col] = v[c][r] * sv[c];
    }
  }
  };
  run_pass(std::integral_constant<int, 0>{});
  if (a.tail && !a.fold) run_pass(std::integral_constant<int, 1>{});
}

// Merges a split tail's partials: one wavefront per query row of a
// leftover block (plane p, leftover j, row), lane L holding coordinates L
// and L + 64: the upp partials by their running maxima, 1/l, then
// R_v^T = diag(s_v) H / sqrt(d).
__global__ __launch_bounds__(256) void chunk_tail_merge_kernel(ChunkArgs a, int planes) {
  const int L = threadIdx.x & 63;
  const int w = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (w >= planes * a.tail_r * kQB) return;
  const int row = w % kQB, j = (w / kQB) % a.tail_r, p = w / (kQB * a.tail_r);
  const int gb = p * a.bpp + kCWaves * a.upp + j;
  const int bh = gb / a.qb, q = (gb % a.qb) * kQB + row;
  if (q >= a.Tq) return;
  const int parts = a.upp * a.nsub;
  const size_t r0 = ((size_t)p * a.tail_r + j) * parts;        // partial k: row (r0 + k) 32 + row
  // every partial's maximum in one lane (upp nsub <= 64 by the plan)
  const float2 mlL = L < parts ? a.tail_ml[(r0 + L) * kQB + row] : make_float2(-INFINITY, 0.0f);
  const float M = wave_max(mlL.x);
  const int c0 = a.vperm ? part_pos(L) : L, c1 = a.vperm ? part_pos(L + 64) : L + 64;
  float lsum = 0.0f, x0 = 0.0f, x1 = 0.0f;
  if (M != -INFINITY) {                // the same in every lane
    const float f = mlL.x == -INFINITY ? 0.0f : exp2f(mlL.x - M);
    lsum = wave_sum(f * mlL.y);
    // eight partials' loads in flight at a time (a partial past the last
    // reads the last one again and is weighted by zero)
    for (int k0 = 0; k0 < parts; k0 += 8) {
      float v0[8], v1[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float* o = a.tail_o + ((r0 + min(k0 + u, parts - 1)) * kQB + row) * kHeadDim;
        v0[u] = o[c0];
        v1[u] = o[c1];
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float fk = k0 + u < parts ? __shfl(f, k0 + u, 64) : 0.0f;
        x0 = fmaf(fk, v0[u], x0);
        x1 = fmaf(fk, v1[u], x1);
      }
    }
  }
  const float inv = lsum > 0.0f ? 1.0f / lsum : 0.0f;
  x0 *= inv;
  x1 *= inv;
  wht128(x0, x1);
  float* dst = a.out + ((size_t)bh * a.Tq + q) * kHeadDim;
  dst[L] = x0 * kInvSqrtD * splitmix_sign(a.vseed, L);
  dst[L + 64] = x1 * kInvSqrtD * splitmix_sign(a.vseed, L + 64);
}

struct ChunkPlan {
  int Tc_pad;
  int qb, bpp, packed;
  int tail, upp, tail_r, fold, nsub;   // split tails (see ChunkArgs)
  size_t k_off, v_off, to_off, tml_off, total;
};

// The blocks of a call and their workgroups; the workspace: the current
// chunk's rotated key rows and value rows (padded to whole tiles), which
// every workgroup of a plane reads, and the split
// tails' partials.  The queries are rotated inside the attention kernel, and
// nothing of the cached window is staged.  Split tails are taken when a
// plane has at least two workgroups of whole blocks and one to four blocks
// over: a leftover block then adds a share of the tiles to each of the
// plane's workgroups instead of a second plane's decoding to a workgroup
// that spans two planes.
ChunkPlan chunk_plan(int B, int Hq, int Hkv, int Tq, int Tc, bool corr) {
  (void)corr;
  ChunkPlan p;
  p.Tc_pad = (Tc + kCurPad - 1) / kCurPad * kCurPad;
  p.qb = (Tq + kQB - 1) / kQB;
  p.bpp = (Hq / Hkv) * p.qb;
  p.packed = p.bpp >= kCWaves;
  p.upp = p.bpp / kCWaves;
  p.tail_r = p.bpp % kCWaves;
  p.tail = p.packed && p.upp >= 2 && p.upp <= 64 && p.tail_r >= 1 && p.tail_r <= 4;
  p.fold = p.tail && p.tail_r <= 2 && p.upp * (4 / (2 * p.tail_r)) <= 64;
  p.nsub = p.fold ? 4 / (2 * p.tail_r) : 1;
  const size_t row = kHeadDim * sizeof(_Float16);
  auto up = [](size_t n) { return (n + 255) / 256 * 256; };
  p.k_off = 0;
  const size_t kv = (size_t)B * Hkv * p.Tc_pad * row;
  p.v_off = p.k_off + up(kv);
  p.to_off = p.v_off + up(kv);
  const size_t tail_rows = p.tail ? (size_t)B * Hkv * p.tail_r * p.upp * p.nsub * kQB : 0;
  p.tml_off = p.to_off + up(tail_rows * kHeadDim * sizeof(float));
  p.total = std::max<size_t>(p.tml_off + up(tail_rows * sizeof(float2)), 256);
  return p;
}

// The kernel's view of a codec; its table space is assigned by the caller.
ChunkCodec chunk_codec(const Codec& c) {
  ChunkCodec k;
  std::memset(&k, 0, sizeof(k));
  k.sel = c.group ? 1000 + 100 * c.bits + c.group : 10 * c.b_dir + c.b_nrm;
  k.W = c.w_idx;
  return k;
}

// The attention kernel for a codec pair: compiled for the pair when keys and
// values use the same codec (the common case: the word registers and the
// decoders are then fixed), else the one that chooses the codecs at run time.
const void* chunk_kernel(bool corr, int ksel, int vsel) {
  if (ksel == vsel) {
#define K_(C, S) case S: return reinterpret_cast<const void*>(&chunk_attn_kernel<C, S, S>);
    if (corr) {
      switch (ksel) { K_(true, 1216) K_(true, 1232) K_(true, 1316) K_(true, 1332) K_(true, 1416) K_(true, 1432) }
    } else {
      switch (ksel) {
        K_(false, 31) K_(false, 42) K_(false, 53) K_(false, 22) K_(false, 33) K_(false, 44)
        K_(false, 1216) K_(false, 1232) K_(false, 1316) K_(false, 1332) K_(false, 1416) K_(false, 1432)
      }
    }
#undef K_
  }
  return corr ? reinterpret_cast<const void*>(&chunk_attn_kernel<true, 0, 0>)
              : reinterpret_cast<const void*>(&chunk_attn_kernel<false, 0, 0>);
}

// LDS bytes of an OCTOPUS codec's table in its copies (and rho pairs).
int table_bytes(const Codec& c, int* rho_off) {
  const int entries = pre_entries(c.b_dir, c.b_nrm);
  const int tab = entries * 8 * tab_copies(c.b_dir, c.b_nrm);
  *rho_off = tab;
  return entries == c.K * c.K * c.R ? tab : tab + c.R * 4;
}

}  // namespace
}  // namespace octo

using namespace octo;

extern "C" octo_status octo_chunk_workspace_bytes(const octo_codec_desc* k_codec, int32_t B,
                                                  int32_t num_q_heads, int32_t kv_heads,
                                                  int32_t Tq, int32_t cached_tokens, int32_t Tc,
                                                  uint32_t flags, size_t* bytes) {
  clear_error();
  Codec kc;
  octo_status s = resolve_codec(k_codec, "octo_chunk_workspace_bytes", &kc, false);
  if (s != OCTO_OK) return s;
  if (flags & ~OCTO_CHUNK_JENSEN_CORRECTION)
    return fail(OCTO_ERR_INVALID_ARGUMENT, "octo_chunk_workspace_bytes: unknown flags 0x%x", flags);
  if (!bytes) return fail(OCTO_ERR_INVALID_ARGUMENT, "octo_chunk_workspace_bytes: bytes is NULL");
  if (B < 1 || num_q_heads < 1 || kv_heads < 1 || Tq < 0 || cached_tokens < 0 || Tc < 0)
    return fail(OCTO_ERR_INVALID_ARGUMENT, "octo_chunk_workspace_bytes: bad sizes");
  *bytes = chunk_plan(B, num_q_heads, kv_heads, Tq, Tc, (flags & OCTO_CHUNK_JENSEN_CORRECTION) != 0).total;
  return OCTO_OK;
}

extern "C" octo_status octo_attend_chunk(const octo_codec_desc* k_codec,
                                         const octo_codec_desc* v_codec,
                                         const octo_cache_view* k_cache,
                                         const octo_cache_view* v_cache, int32_t cached_tokens,
                                         const void* q, const void* k_cur, const void* v_cur,
                                         int32_t num_q_heads, int32_t Tq, int32_t Tc,
                                         float softmax_scale, uint32_t flags, float* out,
                                         void* workspace, size_t workspace_bytes,
                                         hipStream_t stream) {
  clear_error();
  const char* what = "octo_attend_chunk";
  Codec kc, vc;
  octo_status s;
  if ((s = resolve_codec(k_codec, what, &kc)) != OCTO_OK) return s;
  if ((s = resolve_codec(v_codec, what, &vc)) != OCTO_OK) return s;
  if ((s = check_cache(k_cache, kc, what)) != OCTO_OK) return s;
  if ((s = check_cache(v_cache, vc, what)) != OCTO_OK) return s;
  if (kc.qjl || vc.qjl) return fail(OCTO_ERR_UNSUPPORTED, "%s: QJL is not supported here", what);
  if (flags & ~OCTO_CHUNK_JENSEN_CORRECTION)
    return fail(OCTO_ERR_INVALID_ARGUMENT, "%s: unknown flags 0x%x", what, flags);
  const bool corr = (flags & OCTO_CHUNK_JENSEN_CORRECTION) != 0;
  if (corr && !kc.group)
    return fail(OCTO_ERR_UNSUPPORTED,
                "%s: the Jensen-bias correction models round-to-nearest keys (group codec)", what);
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
  // the rows are read 16 bytes a lane
  if (((uintptr_t)q | (uintptr_t)k_cur | (uintptr_t)v_cur) & 15 || ((uintptr_t)out & 3))
    return fail(OCTO_ERR_ALIGNMENT, "%s: q, k_cur, v_cur (16 bytes) or out (4) misaligned", what);
  const ChunkPlan p = chunk_plan(B, num_q_heads, Hkv, Tq, Tc, corr);
  // buffer descriptors address a plane's current rows and packed streams
  // with 32-bit byte ranges
  if ((int64_t)p.Tc_pad * kVSrcBytes > INT32_MAX ||
      (int64_t)k_cache->capacity * std::max(kc.w_idx, vc.w_idx) * 4 > INT32_MAX)
    return fail(OCTO_ERR_UNSUPPORTED, "%s: a plane's rows or packed streams exceed 2 GiB", what);
  if (!workspace || workspace_bytes < p.total)
    return fail(OCTO_ERR_WORKSPACE_TOO_SMALL, "%s: workspace %zu bytes, need %zu", what,
                workspace_bytes, p.total);
  if ((uintptr_t)workspace & 255)
    return fail(OCTO_ERR_ALIGNMENT, "%s: workspace must be 256-byte aligned", what);

  char* ws = static_cast<char*>(workspace);
  _Float16* kr = reinterpret_cast<_Float16*>(ws + p.k_off);
  _Float16* vr = reinterpret_cast<_Float16*>(ws + p.v_off);
  const int planes_kv = B * Hkv;
  // coordinates in part order for tensors in the OCTOPUS codec (queries and
  // current keys follow the keys' codec)
  const int kperm = kc.group ? 0 : 1, vperm = vc.group ? 0 : 1;

  const float tau = softmax_scale > 0.0f ? softmax_scale : kInvSqrtD;
  const float scale2 = tau * kLog2e;
  // query features: minus 16 log2(e) tau^2 / 24 ||(R q)_j||^2 (the key
  // features carry Delta^2 / 16), so that their product is -b in log2 units
  const float feat_c = -16.0f * kLog2e * tau * tau / 24.0f;
  // the pre-pass: the current keys and values
  const int cur_tiles = (p.Tc_pad + 63) / 64;
  RotJob jk{static_cast<const uint16_t*>(k_cur), Tc, p.Tc_pad, kc.seed, kr, p.Tc_pad, kHeadDim,
            cur_tiles, planes_kv, kperm};
  RotJob jv{static_cast<const uint16_t*>(v_cur), Tc, p.Tc_pad, vc.seed, vr, p.Tc_pad, kHeadDim,
            cur_tiles, planes_kv, vperm};
  const long rot_blocks = Tc > 0 ? (long)cur_tiles * planes_kv * 2 : 0;
  if (rot_blocks > 0)
    hipLaunchKernelGGL(rotate_rows_kernel, dim3((unsigned)rot_blocks), dim3(256), 0, stream, jk, jv);
  if ((s = check_launch(what)) != OCTO_OK) return s;

  ChunkArgs a;
  std::memset(&a, 0, sizeof(a));
  a.q = static_cast<const uint16_t*>(q);
  a.kseed = kc.seed;
  a.q_post = kInvSqrtD * scale2;
  a.kperm = kperm;
  a.feat_c = feat_c;
  a.feat_gs = corr ? kc.group : 32;
  a.kc = kr;
  a.vc = vr;
  a.out = out;
  a.Hq = num_q_heads;
  a.Hkv = Hkv;
  a.Tq = Tq;
  a.qb = p.qb;
  const long long n_blocks = (long long)B * num_q_heads * a.qb;
  if (n_blocks > 0x7fffffffLL) return fail(OCTO_ERR_UNSUPPORTED, "%s: too many query blocks", what);
  a.n_blocks = (int)n_blocks;
  a.bpp = p.bpp;
  a.packed = p.packed;
  a.tail = p.tail;
  a.upp = p.upp;
  a.tail_r = p.tail_r;
  a.fold = p.fold;
  a.nsub = p.nsub;
  a.tail_tt = 0;
  if (p.tail) {
    const int n_tiles = (cached_tokens + kBN - 1) / kBN + (Tc + kBN - 1) / kBN;
    a.tail_tt = (n_tiles + p.upp - 1) / p.upp;
    a.tail_o = reinterpret_cast<float*>(ws + p.to_off);
    a.tail_ml = reinterpret_cast<float2*>(ws + p.tml_off);
  }
  a.cached = cached_tokens;
  a.Tc = Tc;
  a.Tc_pad = p.Tc_pad;
  a.capacity = k_cache->capacity;
  a.vseed = vc.seed;
  a.k_idx = k_cache->idx;
  a.v_idx = v_cache->idx;
  a.k_gamma = k_cache->gamma;
  a.v_gamma = v_cache->gamma;
  a.kcod = chunk_codec(kc);
  a.vcod = chunk_codec(vc);
  a.vperm = vperm;
  a.kcb = kc.cb;
  a.vcb = vc.cb;
  // dynamic LDS: the tables (OCTOPUS codecs)
  int off = 0;
  a.share_tab = !kc.group && !vc.group && kc.b_dir == vc.b_dir && kc.b_nrm == vc.b_nrm &&
                std::memcmp(&kc.cb, &vc.cb, sizeof(Codebook)) == 0;
  if (!kc.group) {
    int rho;
    a.kcod.tab = off;
    off += table_bytes(kc, &rho);
    a.kcod.rho = a.kcod.tab + rho;
  }
  if (!vc.group) {
    if (a.share_tab) {
      a.vcod.tab = a.kcod.tab;
      a.vcod.rho = a.kcod.rho;
    } else {
      int rho;
      a.vcod.tab = (off + 7) / 8 * 8;
      off = a.vcod.tab + table_bytes(vc, &rho);
      a.vcod.rho = a.vcod.tab + rho;
    }
  }
  const size_t dyn_bytes = (size_t)(off + 15) / 16 * 16;
  const long long units = a.tail ? (long long)B * Hkv * a.upp
                                 : a.packed ? (n_blocks + kCWaves - 1) / kCWaves : (long long)B * Hkv;
  const void* fn = chunk_kernel(corr, a.kcod.sel, a.vcod.sel);
  if (dyn_bytes > 65536) {
    const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)dyn_bytes);
    if (e != hipSuccess) return fail(OCTO_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  }
  void* kargs[] = {&a};
  hipError_t e = hipLaunchKernel(fn, dim3((unsigned)units), dim3(kCThreads), kargs, dyn_bytes, stream);
  if (e != hipSuccess) return fail(OCTO_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  if ((s = check_launch(what)) != OCTO_OK) return s;
  if (a.tail) {
    // the leftover blocks' rows, four a workgroup
    const long long rows = (long long)B * Hkv * a.tail_r * kQB;
    hipLaunchKernelGGL(chunk_tail_merge_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, stream,
                       a, B * Hkv);
    return check_launch(what);
  }
  return OCTO_OK;
}
